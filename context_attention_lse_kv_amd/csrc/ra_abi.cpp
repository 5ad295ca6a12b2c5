// C ABI of the ring-attention library: host-side validation (before any
// launch), chunk-table and ring-order handling, workspace carving and the
// launch sequence of the ring sweeps.  Everything is enqueued on the caller's
// stream; nothing here allocates device memory.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "ra_internal.h"

namespace {

thread_local std::string g_err;

ra_status fail(ra_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

ra_status ok() {
    g_err.clear();
    return RA_OK;
}

#define RA_TRY(expr)                      \
    do {                                  \
        const ra_status _st = (expr);     \
        if (_st != RA_OK) return _st;     \
    } while (0)

#define RA_HIP(expr)                                                                  \
    do {                                                                              \
        const hipError_t _e = (expr);                                                 \
        if (_e != hipSuccess) return fail(RA_E_HIP, "%s: %s", #expr, hipGetErrorString(_e)); \
    } while (0)

size_t esize(int32_t dt) { return dt == RA_BF16 ? 2 : dt == RA_F32 ? 4 : 0; }
const char* dname(int32_t dt) { return dt == RA_BF16 ? "bf16" : dt == RA_F32 ? "fp32" : "invalid"; }

int64_t numel(const ra_tensor& t) { return (int64_t)t.B * t.S * t.H * t.D; }

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

// True if no two logical elements of the tensor share an address (trivially so for a
// tensor with no elements, whatever its strides).
bool non_overlapping(const ra_tensor& t) {
    if (numel(t) == 0) return true;
    struct Dim { int64_t stride, extent; };
    std::vector<Dim> dims = {{1, t.D}, {t.sH, t.H}, {t.sS, t.S}, {t.sB, t.B}};
    dims.erase(std::remove_if(dims.begin(), dims.end(), [](const Dim& d) { return d.extent <= 1; }), dims.end());
    std::sort(dims.begin(), dims.end(), [](const Dim& a, const Dim& b) { return a.stride < b.stride; });
    int64_t span = 0;  // largest offset reachable by the inner dims
    for (const Dim& d : dims) {
        if (d.stride <= span) return false;
        span += d.stride * (d.extent - 1);
    }
    return true;
}

// Byte range [lo, hi) that a tensor touches.
void byte_range(const ra_tensor& t, uintptr_t& lo, uintptr_t& hi) {
    const size_t es = esize(t.dtype);
    lo = (uintptr_t)t.data;
    if (numel(t) == 0) {
        hi = lo;
        return;
    }
    const int64_t last = (int64_t)(t.B - 1) * t.sB + (int64_t)(t.S - 1) * t.sS + (int64_t)(t.H - 1) * t.sH + (t.D - 1);
    hi = lo + (uintptr_t)((last + 1) * es);
}

ra_status check_tensor(const ra_tensor* t, const char* name, bool any_d = false) {
    if (!t) return fail(RA_E_ARG, "%s: descriptor is NULL", name);
    const size_t es = esize(t->dtype);
    if (es == 0) return fail(RA_E_DTYPE, "%s: dtype %d is neither RA_BF16 nor RA_F32", name, t->dtype);
    if (t->B < 1 || t->H < 1 || t->D < 1 || t->S < 0)
        return fail(RA_E_SHAPE, "%s: need B, H, D >= 1 and S >= 0 (got B=%d S=%d H=%d D=%d)", name, t->B, t->S,
                    t->H, t->D);
    if (!any_d && t->D != 64 && t->D != 128)
        return fail(RA_E_UNSUPPORTED, "%s: head dim D=%d is not built (D must be 64 or 128)", name, t->D);
    if (any_d && (t->D * es) % 16 != 0)
        return fail(RA_E_ALIGN, "%s: a row of D=%d %s elements is not a multiple of 16 bytes", name, t->D,
                    dname(t->dtype));
    if (t->sB < 0 || t->sS < 0 || t->sH < 0) return fail(RA_E_ARG, "%s: negative stride", name);
    if (numel(*t) > 0 && !t->data) return fail(RA_E_ARG, "%s: data is NULL", name);
    if ((uintptr_t)t->data % 16) return fail(RA_E_ALIGN, "%s: data pointer is not 16-byte aligned", name);
    if ((t->sB * es) % 16 || (t->sS * es) % 16 || (t->sH * es) % 16)
        return fail(RA_E_ALIGN, "%s: strides (%lld, %lld, %lld) elements are not multiples of 16 bytes", name,
                    (long long)t->sB, (long long)t->sS, (long long)t->sH);
    if (!non_overlapping(*t)) return fail(RA_E_ARG, "%s: strides make elements overlap", name);
    return RA_OK;
}

ra_status check_rows(const ra_lse* l, const char* name, int32_t B, int32_t H, int32_t S) {
    if (!l) return fail(RA_E_ARG, "%s: descriptor is NULL", name);
    if (l->B != B || l->H != H || l->S != S)
        return fail(RA_E_SHAPE, "%s: shape [%d,%d,%d] does not match [B,H,S]=[%d,%d,%d]", name, l->B, l->H, l->S, B,
                    H, S);
    if (l->sB < 0 || l->sH < 0) return fail(RA_E_ARG, "%s: negative stride", name);
    if ((int64_t)B * H * S > 0 && !l->data) return fail(RA_E_ARG, "%s: data is NULL", name);
    if ((uintptr_t)l->data % 4) return fail(RA_E_ALIGN, "%s: data pointer is not 4-byte aligned", name);
    if (S > 1 || H > 1 || B > 1) {
        // rows of the statistic must not overlap: sH >= S (when H > 1) and sB >= (H-1)*sH + S (when B > 1)
        if (H > 1 && l->sH < S) return fail(RA_E_ARG, "%s: sH < S makes rows overlap", name);
        if (B > 1 && l->sB < (int64_t)(H - 1) * l->sH + S) return fail(RA_E_ARG, "%s: sB makes rows overlap", name);
    }
    return RA_OK;
}

// The bf16 kernels address one (batch, head) slice with 32-bit buffer offsets: the
// slice's byte span, plus one tile of slack, must stay below 2^31.
ra_status check_span32(const ra_tensor& t, const char* name) {
    const int64_t span = ((int64_t)(t.S + 128) * t.sS + t.D) * (int64_t)esize(t.dtype);
    if (span >= ((int64_t)1 << 31))
        return fail(RA_E_UNSUPPORTED, "%s: one (batch, head) slice spans %lld bytes; the bf16 kernels need < 2^31",
                    name, (long long)span);
    return RA_OK;
}

bool same_shape(const ra_tensor& a, const ra_tensor& b) { return a.B == b.B && a.S == b.S && a.H == b.H && a.D == b.D; }

ra_status check_scale(float scale) {
    // lower bound: the dK/dV kernel forms -lse / scale, which must stay finite
    if (!std::isfinite(scale) || !(scale >= 0x1p-100f)) return fail(RA_E_ARG, "scale must be finite and >= 2^-100 (got %g)", scale);
    return RA_OK;
}

// q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D] with matching dtype, batch and head dim, Hkv | Hq.
ra_status check_qkv(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v) {
    RA_TRY(check_tensor(q, "q"));
    RA_TRY(check_tensor(k, "k"));
    RA_TRY(check_tensor(v, "v"));
    if (q->dtype != k->dtype || q->dtype != v->dtype)
        return fail(RA_E_DTYPE, "q, k, v must share one dtype (got %s, %s, %s)", dname(q->dtype), dname(k->dtype),
                    dname(v->dtype));
    if (k->B != q->B || v->B != q->B) return fail(RA_E_SHAPE, "batch of q, k, v differs");
    if (k->D != q->D || v->D != q->D) return fail(RA_E_SHAPE, "head dim of q, k, v differs");
    if (k->S != v->S || k->H != v->H) return fail(RA_E_SHAPE, "k and v must have the same sequence length and heads");
    if (q->H % k->H != 0)
        return fail(RA_E_SHAPE,
                    "Number of heads in key/value must divide number of heads in query (H_q=%d, H_kv=%d)", q->H, k->H);
    if (q->dtype == RA_BF16) {
        RA_TRY(check_span32(*q, "q"));
        RA_TRY(check_span32(*k, "k"));
        RA_TRY(check_span32(*v, "v"));
    }
    return RA_OK;
}

ra_status check_acc(const ra_tensor* t, const char* name, const ra_tensor& like) {
    RA_TRY(check_tensor(t, name));
    if (t->dtype != RA_F32) return fail(RA_E_DTYPE, "%s: accumulator must be fp32", name);
    if (!same_shape(*t, like)) return fail(RA_E_SHAPE, "%s: shape does not match", name);
    return RA_OK;
}

ra_status check_chunks(const ra_chunks* c, int32_t Sk) {
    if (!c) return fail(RA_E_ARG, "chunks: descriptor is NULL");
    if (c->n < 1 || c->n > 65536) return fail(RA_E_ARG, "chunks: n=%d out of range [1, 65536]", c->n);
    if (!c->start || !c->len || !c->order) return fail(RA_E_ARG, "chunks: start/len/order must not be NULL");
    std::vector<int> seen(c->n, 0);
    for (int i = 0; i < c->n; ++i) {
        const int o = c->order[i];
        if (o < 0 || o >= c->n || seen[o]++) return fail(RA_E_ARG, "chunks: order is not a permutation of 0..n-1");
    }
    std::vector<std::pair<int64_t, int64_t>> iv;
    for (int i = 0; i < c->n; ++i) {
        if (c->len[i] < 0 || c->start[i] < 0) return fail(RA_E_ARG, "chunks: negative start or length");
        if ((int64_t)c->start[i] + c->len[i] > Sk)
            return fail(RA_E_SHAPE, "chunks: chunk %d [%d, %d) runs past S_k=%d", i, c->start[i],
                        c->start[i] + c->len[i], Sk);
        if (c->len[i] > 0) iv.push_back({c->start[i], c->len[i]});
    }
    std::sort(iv.begin(), iv.end());
    int64_t at = 0;
    for (auto& x : iv) {
        if (x.first != at) return fail(RA_E_SHAPE, "chunks do not tile [0, S_k) exactly (gap or overlap at %lld)", (long long)at);
        at += x.second;
    }
    if (at != Sk) return fail(RA_E_SHAPE, "chunks cover %lld of S_k=%d rows", (long long)at, Sk);
    return RA_OK;
}

ra_tensor seq_slice(const ra_tensor& t, int32_t start, int32_t len) {
    ra_tensor r = t;
    r.data = (char*)t.data + (int64_t)start * t.sS * (int64_t)esize(t.dtype);
    r.S = len;
    return r;
}

ra_tensor contiguous_f32(void* data, const ra_tensor& like) {
    ra_tensor r;
    r.data = data;
    r.dtype = RA_F32;
    r.B = like.B; r.S = like.S; r.H = like.H; r.D = like.D;
    r.sH = like.D;
    r.sS = (int64_t)like.H * like.D;
    r.sB = (int64_t)like.S * like.H * like.D;
    return r;
}

ra_lse contiguous_rows(void* data, int32_t B, int32_t H, int32_t S) {
    ra_lse r;
    r.data = (float*)data;
    r.B = B; r.H = H; r.S = S;
    r.sH = S;
    r.sB = (int64_t)H * S;
    return r;
}

// Validation of an optional key mask over S keys of B batches (NULL = no mask).
ra_status check_kmask(const ra_kmask* m, int32_t B, int32_t S) {
    if (!m) return RA_OK;
    if (m->B != B || m->S != S)
        return fail(RA_E_SHAPE, "kmask: shape [%d,%d] does not match [B,S_k]=[%d,%d]", m->B, m->S, B, S);
    if (m->sB < 0) return fail(RA_E_ARG, "kmask: negative stride");
    if (B > 1 && m->sB < S) return fail(RA_E_ARG, "kmask: sB < S makes rows overlap");
    if ((int64_t)B * S > 0 && !m->data) return fail(RA_E_ARG, "kmask: data is NULL");
    return RA_OK;
}

// The kernels' view of the mask rows [start, start + len) of every batch.
ra::KeyMask key_mask(const ra_kmask* m, int32_t start = 0) {
    ra::KeyMask r;
    r.data = m ? m->data + start : nullptr;
    r.sB = m ? m->sB : 0;
    return r;
}

ra_status enqueue_fwd_chunk(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const ra::KeyMask& km,
                            float scale, const ra_tensor& out, const ra_lse& lse, int merge, hipStream_t s,
                            const ra_tensor* out16 = nullptr) {
    if (k.S == 0) {
        if (!merge) {  // the partial of an empty chunk is the merge identity
            RA_HIP(ra::launch_zero_f32(out, s));
            RA_HIP(ra::launch_fill_rows(lse, -INFINITY, s));
        }
        return RA_OK;
    }
    if (q.dtype == RA_BF16) RA_HIP(ra::launch_fwd_chunk_bf16(q, k, v, km, scale, out, lse, merge, s, out16));
    else RA_HIP(ra::launch_fwd_chunk_f32(q, k, v, km, scale, out, lse, merge, s));
    return RA_OK;
}

ra_status enqueue_bwd_dkdv(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const ra_tensor& dout,
                           const ra_lse& lse, const ra_lse& delta, const ra::KeyMask& km, float scale,
                           const ra_tensor& dk, const ra_tensor& dv, hipStream_t s) {
    if (q.dtype == RA_BF16) RA_HIP(ra::launch_bwd_dkdv_bf16(q, k, v, dout, lse, delta, km, scale, dk, dv, nullptr, s));
    else RA_HIP(ra::launch_bwd_dkdv_f32(q, k, v, dout, lse, delta, km, scale, dk, dv, s));
    return RA_OK;
}

ra_status enqueue_bwd_dq(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const ra_tensor& dout,
                         const ra_lse& lse, const ra_lse& delta, const ra::KeyMask& km, float scale,
                         const ra_tensor& dq, hipStream_t s) {
    if (q.dtype == RA_BF16) RA_HIP(ra::launch_bwd_dq_bf16(q, k, v, dout, lse, delta, km, scale, dq, s));
    else RA_HIP(ra::launch_bwd_dq_f32(q, k, v, dout, lse, delta, km, scale, dq, s));
    return RA_OK;
}

ra_status enqueue_bwd_chunk(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const ra_tensor& dout,
                            const ra_lse& lse, const ra_lse& delta, const ra::KeyMask& km, float scale,
                            const ra_tensor& dq, const ra_tensor& dk, const ra_tensor& dv, hipStream_t s) {
    RA_TRY(enqueue_bwd_dkdv(q, k, v, dout, lse, delta, km, scale, dk, dv, s));
    RA_TRY(enqueue_bwd_dq(q, k, v, dout, lse, delta, km, scale, dq, s));
    return RA_OK;
}

// Shared validation of the backward chunk entry points (accumulators may be NULL when
// the entry point does not touch them).
ra_status check_bwd_chunk(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const ra_tensor* dout,
                          const ra_lse* lse, const ra_lse* delta, float scale) {
    RA_TRY(check_qkv(q, k, v));
    RA_TRY(check_tensor(dout, "dout"));
    if (dout->dtype != q->dtype) return fail(RA_E_DTYPE, "dout must have the dtype of q");
    if (!same_shape(*dout, *q)) return fail(RA_E_SHAPE, "dout must have the shape of q");
    // dout may have strides of its own: its slices get the same 32-bit bound as q's
    if (q->dtype == RA_BF16) RA_TRY(check_span32(*dout, "dout"));
    RA_TRY(check_rows(lse, "lse", q->B, q->H, q->S));
    RA_TRY(check_rows(delta, "delta", q->B, q->H, q->S));
    RA_TRY(check_scale(scale));
    return RA_OK;
}

}  // namespace

extern "C" {

ra_status ra_fwd_chunk_masked(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const ra_kmask* kmask,
                              float scale, ra_tensor* out, ra_lse* lse, int32_t merge, void* stream) {
    RA_TRY(check_qkv(q, k, v));
    RA_TRY(check_acc(out, "out", *q));
    RA_TRY(check_rows(lse, "lse", q->B, q->H, q->S));
    RA_TRY(check_scale(scale));
    RA_TRY(check_kmask(kmask, q->B, k->S));
    if (merge != 0 && merge != 1) return fail(RA_E_ARG, "merge must be 0 or 1");
    RA_TRY(enqueue_fwd_chunk(*q, *k, *v, key_mask(kmask), scale, *out, *lse, merge, (hipStream_t)stream));
    return ok();
}

ra_status ra_fwd_chunk(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, float scale, ra_tensor* out,
                       ra_lse* lse, int32_t merge, void* stream) {
    return ra_fwd_chunk_masked(q, k, v, nullptr, scale, out, lse, merge, stream);
}

ra_status ra_merge_lse(ra_tensor* out_acc, ra_lse* lse_acc, const ra_tensor* out_part, const ra_lse* lse_part,
                       void* stream) {
    RA_TRY(check_tensor(out_acc, "out_acc"));
    RA_TRY(check_acc(out_part, "out_part", *out_acc));
    if (out_acc->dtype != RA_F32) return fail(RA_E_DTYPE, "out_acc must be fp32");
    RA_TRY(check_rows(lse_acc, "lse_acc", out_acc->B, out_acc->H, out_acc->S));
    RA_TRY(check_rows(lse_part, "lse_part", out_acc->B, out_acc->H, out_acc->S));
    RA_HIP(ra::launch_merge_lse(*out_acc, *lse_acc, *out_part, *lse_part, (hipStream_t)stream));
    return ok();
}

ra_status ra_bwd_delta(const ra_tensor* out, const ra_tensor* dout, ra_lse* delta, void* stream) {
    RA_TRY(check_tensor(out, "out"));
    RA_TRY(check_tensor(dout, "dout"));
    if (!same_shape(*out, *dout)) return fail(RA_E_SHAPE, "out and dout must have the same shape");
    if (out->dtype == RA_BF16 && dout->dtype == RA_F32)
        return fail(RA_E_DTYPE, "bf16 out with fp32 dout is not supported");
    RA_TRY(check_rows(delta, "delta", out->B, out->H, out->S));
    RA_HIP(ra::launch_bwd_delta(*out, *dout, *delta, (hipStream_t)stream));
    return ok();
}

ra_status ra_bwd_chunk_masked(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const ra_tensor* dout,
                              const ra_lse* lse, const ra_lse* delta, const ra_kmask* kmask, float scale,
                              ra_tensor* dq_acc, ra_tensor* dk_acc, ra_tensor* dv_acc, int32_t accumulate,
                              void* stream) {
    RA_TRY(check_bwd_chunk(q, k, v, dout, lse, delta, scale));
    RA_TRY(check_kmask(kmask, q->B, k->S));
    RA_TRY(check_acc(dq_acc, "dq_acc", *q));
    RA_TRY(check_acc(dk_acc, "dk_acc", *k));
    RA_TRY(check_acc(dv_acc, "dv_acc", *k));
    if (accumulate != 0 && accumulate != 1) return fail(RA_E_ARG, "accumulate must be 0 or 1");
    hipStream_t s = (hipStream_t)stream;
    if (!accumulate) {
        RA_HIP(ra::launch_zero_f32(*dk_acc, s));
        RA_HIP(ra::launch_zero_f32(*dv_acc, s));
    }
    if (k->S > 0 && q->S > 0)
        RA_TRY(enqueue_bwd_chunk(*q, *k, *v, *dout, *lse, *delta, key_mask(kmask), scale, *dq_acc, *dk_acc, *dv_acc, s));
    return ok();
}

ra_status ra_bwd_chunk(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const ra_tensor* dout,
                       const ra_lse* lse, const ra_lse* delta, float scale, ra_tensor* dq_acc, ra_tensor* dk_acc,
                       ra_tensor* dv_acc, int32_t accumulate, void* stream) {
    return ra_bwd_chunk_masked(q, k, v, dout, lse, delta, nullptr, scale, dq_acc, dk_acc, dv_acc, accumulate, stream);
}

ra_status ra_bwd_chunk_dkdv_masked(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const ra_tensor* dout,
                                   const ra_lse* lse, const ra_lse* delta, const ra_kmask* kmask, float scale,
                                   ra_tensor* dk_acc, ra_tensor* dv_acc, int32_t accumulate, void* stream) {
    RA_TRY(check_bwd_chunk(q, k, v, dout, lse, delta, scale));
    RA_TRY(check_kmask(kmask, q->B, k->S));
    RA_TRY(check_acc(dk_acc, "dk_acc", *k));
    RA_TRY(check_acc(dv_acc, "dv_acc", *k));
    if (accumulate != 0 && accumulate != 1) return fail(RA_E_ARG, "accumulate must be 0 or 1");
    hipStream_t s = (hipStream_t)stream;
    if (!accumulate) {
        RA_HIP(ra::launch_zero_f32(*dk_acc, s));
        RA_HIP(ra::launch_zero_f32(*dv_acc, s));
    }
    if (k->S > 0 && q->S > 0)
        RA_TRY(enqueue_bwd_dkdv(*q, *k, *v, *dout, *lse, *delta, key_mask(kmask), scale, *dk_acc, *dv_acc, s));
    return ok();
}

ra_status ra_bwd_chunk_dkdv(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const ra_tensor* dout,
                            const ra_lse* lse, const ra_lse* delta, float scale, ra_tensor* dk_acc,
                            ra_tensor* dv_acc, int32_t accumulate, void* stream) {
    return ra_bwd_chunk_dkdv_masked(q, k, v, dout, lse, delta, nullptr, scale, dk_acc, dv_acc, accumulate, stream);
}

ra_status ra_bwd_chunk_dq_masked(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const ra_tensor* dout,
                                 const ra_lse* lse, const ra_lse* delta, const ra_kmask* kmask, float scale,
                                 ra_tensor* dq_acc, void* stream) {
    RA_TRY(check_bwd_chunk(q, k, v, dout, lse, delta, scale));
    RA_TRY(check_kmask(kmask, q->B, k->S));
    RA_TRY(check_acc(dq_acc, "dq_acc", *q));
    if (k->S > 0 && q->S > 0)
        RA_TRY(enqueue_bwd_dq(*q, *k, *v, *dout, *lse, *delta, key_mask(kmask), scale, *dq_acc, (hipStream_t)stream));
    return ok();
}

ra_status ra_bwd_chunk_dq(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const ra_tensor* dout,
                          const ra_lse* lse, const ra_lse* delta, float scale, ra_tensor* dq_acc, void* stream) {
    return ra_bwd_chunk_dq_masked(q, k, v, dout, lse, delta, nullptr, scale, dq_acc, stream);
}

size_t ra_bwd_ds_bytes(const ra_tensor* q, const ra_tensor* k) {
    if (!q || !k || q->dtype != RA_BF16 || q->S <= 0 || k->S <= 0) return 0;
    return round256((size_t)ra::ds_bytes(q->B, q->H, q->S, k->S));
}

static ra_status check_ds(const ra_tensor& q, const ra_tensor& k, const void* ds, size_t ds_bytes) {
    if (q.dtype != RA_BF16) return fail(RA_E_DTYPE, "the stored-dS route is bf16 only");
    const size_t need = ra_bwd_ds_bytes(&q, &k);
    if (need == 0) return RA_OK;
    // the dQ pass addresses one (batch, head) slab of blocks with 32-bit buffer offsets
    if (ra::ds_bytes(1, 1, q.S, k.S) > ((int64_t)1 << 31))
        return fail(RA_E_UNSUPPORTED, "dS of one (batch, head) spans %lld bytes; the dQ pass needs <= 2^31",
                    (long long)ra::ds_bytes(1, 1, q.S, k.S));
    if (!ds) return fail(RA_E_WORKSPACE, "ds buffer of %zu bytes needed, got NULL", need);
    if ((uintptr_t)ds % 256) return fail(RA_E_ALIGN, "ds buffer must be 256-byte aligned");
    if (ds_bytes < need) return fail(RA_E_WORKSPACE, "ds buffer of %zu bytes needed, got %zu", need, ds_bytes);
    return RA_OK;
}

ra_status ra_bwd_chunk_dkdv_ds(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const ra_tensor* dout,
                               const ra_lse* lse, const ra_lse* delta, const ra_kmask* kmask, float scale,
                               ra_tensor* dk_acc, ra_tensor* dv_acc, int32_t accumulate, void* ds, size_t ds_bytes,
                               void* stream) {
    RA_TRY(check_bwd_chunk(q, k, v, dout, lse, delta, scale));
    RA_TRY(check_kmask(kmask, q->B, k->S));
    if (accumulate != 0 && accumulate != 1) return fail(RA_E_ARG, "accumulate must be 0 or 1");
    // bf16 dk/dv: the step's dK/dV are final and written there (accumulate must be 0)
    const bool direct = dk_acc && dv_acc && dk_acc->dtype == RA_BF16 && dv_acc->dtype == RA_BF16;
    if (direct) {
        RA_TRY(check_tensor(dk_acc, "dk_acc"));
        RA_TRY(check_tensor(dv_acc, "dv_acc"));
        if (!same_shape(*dk_acc, *k) || !same_shape(*dv_acc, *k)) return fail(RA_E_SHAPE, "dk/dv: shape does not match");
        if (accumulate) return fail(RA_E_DTYPE, "bf16 dk/dv are written, not accumulated: accumulate must be 0");
    } else {
        RA_TRY(check_acc(dk_acc, "dk_acc", *k));
        RA_TRY(check_acc(dv_acc, "dv_acc", *k));
    }
    RA_TRY(check_ds(*q, *k, ds, ds_bytes));
    hipStream_t s = (hipStream_t)stream;
    if (!accumulate && !direct) {
        RA_HIP(ra::launch_zero_f32(*dk_acc, s));
        RA_HIP(ra::launch_zero_f32(*dv_acc, s));
    }
    if (k->S > 0 && q->S > 0)
        RA_HIP(ra::launch_bwd_dkdv_bf16(*q, *k, *v, *dout, *lse, *delta, key_mask(kmask), scale, *dk_acc, *dv_acc,
                                        ds, s, direct ? dk_acc : nullptr, direct ? dv_acc : nullptr));
    else if (direct && k->S > 0) {
        return fail(RA_E_UNSUPPORTED, "bf16 dk/dv with no query rows: nothing would write them (use fp32)");
    }
    return ok();
}

ra_status ra_bwd_chunk_dq_ds(const ra_tensor* q, const ra_tensor* k, const void* ds, size_t ds_bytes, float scale,
                             ra_tensor* dq_acc, void* stream) {
    RA_TRY(check_tensor(q, "q"));
    RA_TRY(check_tensor(k, "k"));
    if (q->B != k->B || q->D != k->D) return fail(RA_E_SHAPE, "q and k must agree in B and D");
    if (k->H <= 0 || q->H % k->H) return fail(RA_E_SHAPE, "Number of heads in key/value must divide number of heads in query");
    if (k->dtype != q->dtype) return fail(RA_E_DTYPE, "q and k must have the same dtype");
    RA_TRY(check_scale(scale));
    RA_TRY(check_span32(*k, "k"));
    RA_TRY(check_acc(dq_acc, "dq_acc", *q));
    RA_TRY(check_ds(*q, *k, ds, ds_bytes));
    if (k->S > 0 && q->S > 0) RA_HIP(ra::launch_bwd_dqs_bf16(*q, *k, ds, scale, *dq_acc, (hipStream_t)stream));
    return ok();
}

size_t ra_ring_fwd_workspace_bytes(const ra_tensor* q, const ra_tensor* out) {
    if (!q || !out || out->dtype != RA_BF16) return 0;
    return round256((size_t)numel(*q) * 4);
}

// dS region of the bf16 ring backward that ra_ring_bwd_workspace_bytes recommends: enough
// for every query row against every chunk of a table of up to kDqsMaxChunks chunks, capped
// at kDsBudget.  The sweep
// itself uses whatever room the caller's workspace leaves above the minimum: a chunk whose
// dS does not fit is swept in query-row slices (multiples of 64 rows) that do.
static constexpr int64_t kDsBudget = int64_t(8) << 30;
// a sliced chunk keeps the stored-dS route only while each slice's dQ pass has at least
// this many workgroups (one per compute unit)
static constexpr int64_t kMinSliceWorkgroups = 256;
// the sweep runs slice-major (every chunk's dK/dV on a slice of query rows, then one dQ
// pass over all of them) only with slices of at least this many rows: each dK/dV
// launch then still sweeps as many rows as the video shard's
static constexpr int64_t kMinGroupRows = 4096;

static size_t ds_region_bytes(const ra_tensor& q, const ra_tensor& k) {
    if (q.dtype != RA_BF16 || q.S == 0 || k.S == 0) return 0;
    // dS is stored in whole key tiles per chunk, so a table of n chunks needs up to n - 1 key
    // tiles more than the key sequence taken as one chunk; the room covers that for as many
    // chunks as one dQ pass sweeps, so that any such table runs as one group
    const int64_t full = ra::ds_bytes(q.B, q.H, q.S, k.S) +
                         (ra::kDqsMaxChunks - 1) * ra::ds_bytes(q.B, q.H, q.S, ra::kBwdBlockN);
    return round256((size_t)(full < kDsBudget ? full : kDsBudget));
}

}  // extern "C"

namespace {

// Plan of the ring backward for a given workspace size.  Chunk-major (the default): per
// chunk (in sweep order), the stored-dS route with query slices of `rows` rows, or the
// recompute route (rows = 0).  Slice-major (slice_rows > 0), when the dS of every chunk
// does not fit at once but that of every chunk for a slice of at least kMinGroupRows
// query rows does: each slice runs the dK/dV launches of all chunks, in sweep order, and
// then one dQ pass over their dS that writes the slice's dq rows once (no fp32 dQ
// accumulator read and written per chunk, which costs the chunk-major sweep more than the
// slice-major one's dK/dV accumulation over slices).
// fp32 accumulators are carved from the workspace only for bf16 gradients that need one:
// dK/dV when some chunk is swept in more than one slice (else each chunk's rows are final
// after its one dK/dV launch and are written in bf16 directly), dQ unless one dQ pass
// covers the dS of every chunk for the rows it writes (it then writes the bf16 dq directly).
struct BwdStep {
    int c;
    int32_t rows;
};
struct BwdPlan {
    std::vector<BwdStep> steps;
    bool single = false;     // chunk-major, every chunk in one slice on the stored-dS route
    bool one_group = false;  // ... and one dQ pass covers all of them
    int32_t slice_rows = 0;  // > 0: slice-major with slices of this many query rows
    bool dq_acc = false, dk_acc = false, dv_acc = false;
    size_t delta_b = 0, dq_b = 0, dk_b = 0, dv_b = 0;
    size_t fixed() const {
        return delta_b + (dq_acc ? dq_b : 0) + (dk_acc ? dk_b : 0) + (dv_acc ? dv_b : 0);
    }
};

void plan_steps(BwdPlan& P, const ra_tensor& q, const ra_chunks& ch, int64_t ds_room) {
    P.steps.clear();
    for (int i = 0; i < ch.n; ++i) {
        const int c = ch.order[i];
        if (ch.len[c] == 0 || q.S == 0) continue;
        const int64_t per_tile = q.dtype == RA_BF16 ? ra::ds_bytes(q.B, q.H, 64, ch.len[c]) : 0;
        const int64_t slab_rows = per_tile == 0 ? 0 : 64 * ((int64_t(1) << 31) / ra::ds_bytes(1, 1, 64, ch.len[c]));
        int32_t rows = per_tile == 0 || per_tile > ds_room
                           ? 0
                           : (int32_t)std::min<int64_t>({64 * (ds_room / per_tile), slab_rows, (int64_t)q.S});
        if (rows > 0 && rows < q.S && ra::dqs_workgroups(q.B, q.H, rows) < kMinSliceWorkgroups) rows = 0;
        P.steps.push_back({c, rows});
    }
    P.single = !P.steps.empty();
    for (const BwdStep& st : P.steps) P.single = P.single && st.rows >= q.S;
    int64_t all = 0;
    for (const BwdStep& st : P.steps) all += (int64_t)round256((size_t)ra::ds_bytes(q.B, q.H, q.S, ch.len[st.c]));
    P.one_group = P.single && P.steps.size() <= (size_t)ra::kDqsMaxChunks && all <= ds_room;
    P.slice_rows = 0;
    if (P.one_group || P.steps.empty() || P.steps.size() > (size_t)ra::kDqsMaxChunks) return;
    int64_t per64 = 0, slab = q.S;  // dS of 64 rows against every chunk; 32-bit slab bound
    for (const BwdStep& st : P.steps) {
        if (st.rows == 0) return;  // a chunk on the recompute route
        per64 += ra::ds_bytes(q.B, q.H, 64, ch.len[st.c]);
        slab = std::min<int64_t>(slab, 64 * ((int64_t(1) << 31) / ra::ds_bytes(1, 1, 64, ch.len[st.c])));
    }
    const int64_t rows = std::min<int64_t>(64 * (ds_room / per64), slab);
    if (rows >= kMinGroupRows && rows < q.S) {
        P.slice_rows = (int32_t)rows;
        P.single = false;
    }
}

// The plan for a workspace of ws_bytes (SIZE_MAX: the recommended size, with a dS region
// of ds_region_bytes).  Accumulators are carved first and the dS room is what is left; as
// less room can only need more accumulators, three rounds settle it.
BwdPlan plan_bwd(const ra_tensor& q, const ra_tensor& k, const ra_chunks& ch, const ra_tensor& dq,
                 const ra_tensor& dk, const ra_tensor& dv, size_t ws_bytes) {
    BwdPlan P;
    P.delta_b = round256((size_t)q.B * q.H * q.S * 4);
    P.dq_b = round256((size_t)numel(q) * 4);
    P.dk_b = P.dv_b = round256((size_t)numel(k) * 4);
    const bool rec = ws_bytes == SIZE_MAX;
    for (int round = 0; round < 4; ++round) {
        const size_t f = P.fixed();
        const int64_t room = rec ? (int64_t)ds_region_bytes(q, k)
                                 : (ws_bytes > f ? (int64_t)((ws_bytes - f) & ~(size_t)255) : 0);
        plan_steps(P, q, ch, room);
        const bool ndq = dq.dtype == RA_BF16 && !P.one_group && P.slice_rows == 0;
        const bool nkv = !(P.single && dk.dtype == RA_BF16 && dv.dtype == RA_BF16);
        const bool ndk = dk.dtype == RA_BF16 && nkv, ndv = dv.dtype == RA_BF16 && nkv;
        if ((!ndq || P.dq_acc) && (!ndk || P.dk_acc) && (!ndv || P.dv_acc)) break;
        P.dq_acc |= ndq;
        P.dk_acc |= ndk;
        P.dv_acc |= ndv;
    }
    return P;
}

// Plans for the workspace-size queries, which see no chunk table: the whole key
// sequence as one chunk.
ra_chunks one_chunk(const ra_tensor& k, int32_t* buf) {
    buf[0] = 0;
    buf[1] = k.S;
    buf[2] = 0;
    return ra_chunks{1, &buf[0], &buf[1], &buf[2]};
}

}  // namespace

extern "C" {

size_t ra_ring_bwd_workspace_min_bytes(const ra_tensor* q, const ra_tensor* k, const ra_tensor* dq,
                                       const ra_tensor* dk, const ra_tensor* dv) {
    if (!q || !k) return 0;
    const ra_tensor dq_ = dq ? *dq : *q, dk_ = dk ? *dk : *k, dv_ = dv ? *dv : *k;
    int32_t buf[3];
    const ra_chunks ch = one_chunk(*k, buf);
    const BwdPlan P = plan_bwd(*q, *k, ch, dq_, dk_, dv_, 0);
    return P.fixed();
}

size_t ra_ring_bwd_workspace_bytes(const ra_tensor* q, const ra_tensor* k, const ra_tensor* dq, const ra_tensor* dk,
                                   const ra_tensor* dv) {
    if (!q || !k) return 0;
    const ra_tensor dq_ = dq ? *dq : *q, dk_ = dk ? *dk : *k, dv_ = dv ? *dv : *k;
    int32_t buf[3];
    const ra_chunks ch = one_chunk(*k, buf);
    const BwdPlan P = plan_bwd(*q, *k, ch, dq_, dk_, dv_, SIZE_MAX);
    // never below the size any chunk table is accepted with (a table whose plan needs
    // every accumulator then still runs; accumulators its plan skips become dS room)
    return std::max(P.fixed() + ds_region_bytes(*q, *k), ra_ring_bwd_workspace_min_bytes(q, k, dq, dk, dv));
}

ra_status ra_ring_bwd_plan(const ra_tensor* q, const ra_tensor* k, const ra_tensor* dq, const ra_tensor* dk,
                           const ra_tensor* dv, const ra_chunks* chunks, size_t ws_bytes, int32_t* slice_rows,
                           int32_t* rows, uint32_t* accs) {
    RA_TRY(check_qkv(q, k, k));
    RA_TRY(check_chunks(chunks, k->S));
    const ra_tensor dq_ = dq ? *dq : *q, dk_ = dk ? *dk : *k, dv_ = dv ? *dv : *k;
    for (const ra_tensor* t : {&dq_, &dk_, &dv_})
        if (esize(t->dtype) == 0) return fail(RA_E_DTYPE, "gradient dtype %d is neither RA_BF16 nor RA_F32", t->dtype);
    const BwdPlan P = plan_bwd(*q, *k, *chunks, dq_, dk_, dv_, ws_bytes);
    if (ws_bytes < P.fixed())
        return fail(RA_E_WORKSPACE, "workspace of %zu bytes needed, got %zu", P.fixed(), ws_bytes);
    if (slice_rows) *slice_rows = P.slice_rows;
    if (rows) {
        std::vector<int32_t> by_chunk((size_t)chunks->n, -1);
        for (const BwdStep& st : P.steps) by_chunk[(size_t)st.c] = st.rows > 0 && P.slice_rows > 0 ? P.slice_rows : st.rows;
        for (int i = 0; i < chunks->n; ++i) rows[i] = by_chunk[(size_t)chunks->order[i]];
    }
    if (accs) *accs = (P.dq_acc ? 1u : 0u) | (P.dk_acc ? 2u : 0u) | (P.dv_acc ? 4u : 0u);
    return ok();
}


static ra_lse rows_slice(const ra_lse& t, int32_t start, int32_t len) {
    ra_lse r = t;
    r.data = t.data + start;
    r.S = len;
    return r;
}

static ra_status check_ws(void* ws, size_t ws_bytes, size_t need) {
    if (need == 0) return RA_OK;
    if (!ws) return fail(RA_E_WORKSPACE, "workspace of %zu bytes needed, got NULL", need);
    if ((uintptr_t)ws % 256) return fail(RA_E_ALIGN, "workspace must be 256-byte aligned");
    if (ws_bytes < need) return fail(RA_E_WORKSPACE, "workspace of %zu bytes needed, got %zu", need, ws_bytes);
    return RA_OK;
}

}  // extern "C"

namespace {

ra_status check_ring_fwd(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const ra_kmask* kmask,
                         const ra_chunks* chunks, float scale, const ra_tensor* out, const ra_lse* lse) {
    RA_TRY(check_qkv(q, k, v));
    RA_TRY(check_kmask(kmask, q->B, k->S));
    RA_TRY(check_tensor(out, "out"));
    if (!same_shape(*out, *q)) return fail(RA_E_SHAPE, "out must have the shape of q");
    RA_TRY(check_rows(lse, "lse", q->B, q->H, q->S));
    RA_TRY(check_scale(scale));
    RA_TRY(check_chunks(chunks, k->S));
    return RA_OK;
}

// The forward sweep, validated; ws holds ra_ring_fwd_workspace_bytes(q, out) bytes.
ra_status enqueue_ring_fwd(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const ra_kmask* kmask,
                           const ra_chunks* chunks, float scale, ra_tensor* out, ra_lse* lse, void* ws,
                           hipStream_t s) {
    const ra_tensor acc = out->dtype == RA_F32 ? *out : contiguous_f32(ws, *q);
    // A bf16 sweep's last non-empty step writes the final bf16 output itself (no cast pass).
    int last = -1;
    if (q->dtype == RA_BF16 && out->dtype == RA_BF16 && q->S > 0)
        for (int i = 0; i < chunks->n; ++i)
            if (chunks->len[chunks->order[i]] > 0) last = i;
    for (int i = 0; i < chunks->n; ++i) {
        const int c = chunks->order[i];
        const ra_tensor kc = seq_slice(*k, chunks->start[c], chunks->len[c]);
        const ra_tensor vc = seq_slice(*v, chunks->start[c], chunks->len[c]);
        RA_TRY(enqueue_fwd_chunk(*q, kc, vc, key_mask(kmask, chunks->start[c]), scale, acc, *lse, i > 0 ? 1 : 0, s,
                                 i == last ? out : nullptr));
    }
    if (out->dtype == RA_BF16 && last < 0) RA_HIP(ra::launch_cast_f32_to_bf16(acc, *out, s));
    return RA_OK;
}

}  // namespace

extern "C" {

ra_status ra_ring_fwd_masked(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const ra_kmask* kmask,
                             const ra_chunks* chunks, float scale, ra_tensor* out, ra_lse* lse, void* ws,
                             size_t ws_bytes, void* stream) {
    RA_TRY(check_ring_fwd(q, k, v, kmask, chunks, scale, out, lse));
    RA_TRY(check_ws(ws, ws_bytes, ra_ring_fwd_workspace_bytes(q, out)));
    RA_TRY(enqueue_ring_fwd(q, k, v, kmask, chunks, scale, out, lse, ws, (hipStream_t)stream));
    return ok();
}

ra_status ra_ring_fwd_noalloc(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const ra_kmask* kmask,
                              const ra_chunks* chunks, float scale, ra_tensor* out, ra_lse* lse, void* stream) {
    RA_TRY(check_ring_fwd(q, k, v, kmask, chunks, scale, out, lse));
    const size_t need = ra_ring_fwd_workspace_bytes(q, out);
    if (need > ra::kNoAllocScratchBytes)
        return fail(RA_E_WORKSPACE,
                    "the sweep needs %zu bytes of scratch; ra_ring_fwd_noalloc has %zu (fp32 running output of at most "
                    "%zu elements): use ra_ring_fwd with a workspace",
                    need, ra::kNoAllocScratchBytes, ra::kNoAllocScratchBytes / 4);
    void* ws = nullptr;
    if (need > 0) {
        size_t have = 0;
        RA_HIP(ra::scratch_region(&ws, &have));
    }
    RA_TRY(enqueue_ring_fwd(q, k, v, kmask, chunks, scale, out, lse, ws, (hipStream_t)stream));
    return ok();
}

ra_status ra_ring_fwd(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const ra_chunks* chunks, float scale,
                      ra_tensor* out, ra_lse* lse, void* ws, size_t ws_bytes, void* stream) {
    return ra_ring_fwd_masked(q, k, v, nullptr, chunks, scale, out, lse, ws, ws_bytes, stream);
}

ra_status ra_ring_bwd_masked(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const ra_tensor* out,
                             const ra_tensor* dout, const ra_lse* lse, const ra_kmask* kmask, const ra_chunks* chunks,
                             float scale, ra_tensor* dq, ra_tensor* dk, ra_tensor* dv, void* ws, size_t ws_bytes,
                             void* stream) {
    RA_TRY(check_qkv(q, k, v));
    RA_TRY(check_kmask(kmask, q->B, k->S));
    RA_TRY(check_tensor(out, "out"));
    RA_TRY(check_tensor(dout, "dout"));
    if (!same_shape(*out, *q) || !same_shape(*dout, *q)) return fail(RA_E_SHAPE, "out and dout must have the shape of q");
    if (dout->dtype != q->dtype) return fail(RA_E_DTYPE, "dout must have the dtype of q");
    if (out->dtype == RA_BF16 && dout->dtype == RA_F32) return fail(RA_E_DTYPE, "bf16 out with fp32 dout is not supported");
    if (q->dtype == RA_BF16) RA_TRY(check_span32(*dout, "dout"));
    RA_TRY(check_rows(lse, "lse", q->B, q->H, q->S));
    RA_TRY(check_scale(scale));
    RA_TRY(check_chunks(chunks, k->S));
    RA_TRY(check_tensor(dq, "dq"));
    RA_TRY(check_tensor(dk, "dk"));
    RA_TRY(check_tensor(dv, "dv"));
    if (!same_shape(*dq, *q) || !same_shape(*dk, *k) || !same_shape(*dv, *v))
        return fail(RA_E_SHAPE, "dq, dk, dv must have the shapes of q, k, v");
    const BwdPlan P = plan_bwd(*q, *k, *chunks, *dq, *dk, *dv, ws_bytes);
    RA_TRY(check_ws(ws, ws_bytes, P.fixed()));
    hipStream_t s = (hipStream_t)stream;
    char* p = (char*)ws;
    const ra_lse delta = contiguous_rows(p, q->B, q->H, q->S);
    p += P.delta_b;
    ra_tensor dq_acc = *dq, dk_acc = *dk, dv_acc = *dv;
    if (P.dq_acc) { dq_acc = contiguous_f32(p, *q); p += P.dq_b; }
    if (P.dk_acc) { dk_acc = contiguous_f32(p, *k); p += P.dk_b; }
    if (P.dv_acc) { dv_acc = contiguous_f32(p, *k); p += P.dv_b; }
    void* const ds = p;
    const int64_t ds_room = ws_bytes > P.fixed() ? (int64_t)((ws_bytes - P.fixed()) & ~(size_t)255) : 0;
    const std::vector<BwdStep>& steps = P.steps;
    const bool single = P.single;
    const int32_t slice_rows = P.slice_rows;
    const bool direct_kv = single && dk->dtype == RA_BF16 && dv->dtype == RA_BF16;
    const bool direct_dq = (single || slice_rows > 0) && dq->dtype == RA_BF16;

    RA_HIP(ra::launch_bwd_delta(*out, *dout, delta, s));
    // slice-major: each slice's one dQ pass writes its rows without reading them
    if (!direct_dq && slice_rows == 0) RA_HIP(ra::launch_zero_f32(dq_acc, s));
    if (!direct_kv) {
        RA_HIP(ra::launch_zero_f32(dk_acc, s));
        RA_HIP(ra::launch_zero_f32(dv_acc, s));
    }
    for (int32_t r0 = 0; slice_rows > 0 && r0 < q->S; r0 += slice_rows) {
        // the dK/dV launches of every chunk on rows [r0, r0 + n), their dS stored one
        // after the other, then one dQ pass over all of them
        const int32_t n = std::min(slice_rows, q->S - r0);
        const ra_tensor qs = seq_slice(*q, r0, n), dos = seq_slice(*dout, r0, n);
        const ra_lse ls = rows_slice(*lse, r0, n), dls = rows_slice(delta, r0, n);
        ra::KeyMask kms[ra::kDqsMaxChunks];
        ra::DqsChunk more[ra::kDqsMaxChunks - 1];
        char* dsj = (char*)ds;
        for (size_t j = 0; j < steps.size(); ++j) {
            const int cj = steps[j].c;
            const int32_t st = chunks->start[cj], len = chunks->len[cj];
            const ra_tensor kcj = seq_slice(*k, st, len), vcj = seq_slice(*v, st, len);
            const ra_tensor dkj = seq_slice(dk_acc, st, len), dvj = seq_slice(dv_acc, st, len);
            kms[j] = key_mask(kmask, st);
            RA_HIP(ra::launch_bwd_dkdv_bf16(qs, kcj, vcj, dos, ls, dls, kms[j], scale, dkj, dvj, dsj, s, nullptr,
                                            nullptr));
            if (j > 0) more[j - 1] = ra::DqsChunk{kcj, dsj, kms[j].data ? &kms[j] : nullptr};
            dsj += round256((size_t)ra::ds_bytes(q->B, q->H, n, len));
        }
        const int c0 = steps[0].c;
        const ra_tensor k0 = seq_slice(*k, chunks->start[c0], chunks->len[c0]);
        const ra_tensor dqs = seq_slice(dq_acc, r0, n), dqo = seq_slice(*dq, r0, n);
        RA_HIP(ra::launch_bwd_dqs_bf16(qs, k0, ds, scale, dqs, s, false, direct_dq ? &dqo : nullptr,
                                       kms[0].data ? &kms[0] : nullptr, more, (int)steps.size() - 1));
    }
    for (size_t i = 0; slice_rows == 0 && i < steps.size(); ++i) {
        const int c = steps[i].c;
        const int32_t rows = steps[i].rows;
        const ra_tensor kc = seq_slice(*k, chunks->start[c], chunks->len[c]);
        const ra_tensor vc = seq_slice(*v, chunks->start[c], chunks->len[c]);
        const ra_tensor dkc = seq_slice(dk_acc, chunks->start[c], chunks->len[c]);
        const ra_tensor dvc = seq_slice(dv_acc, chunks->start[c], chunks->len[c]);
        const ra::KeyMask km = key_mask(kmask, chunks->start[c]);
        if (rows == 0) {
            RA_TRY(enqueue_bwd_chunk(*q, kc, vc, *dout, *lse, delta, km, scale, dq_acc, dkc, dvc, s));
            continue;
        }
        // bf16: the dK/dV kernel stores dS, the dQ pass reads it back (no second S, dP)
        const ra_tensor dko = seq_slice(*dk, chunks->start[c], chunks->len[c]);
        const ra_tensor dvo = seq_slice(*dv, chunks->start[c], chunks->len[c]);
        if (single && i + 1 < steps.size()) {
            // Several chunks per dQ pass: the dS of each chunk of the group is stored after
            // the previous one's (as many as the region holds, at most kDqsMaxChunks), and
            // one pass sweeps them all, so the dQ accumulator is read and written once per
            // group instead of once per chunk.
            size_t n = 1;
            int64_t used = (int64_t)round256((size_t)ra::ds_bytes(q->B, q->H, q->S, chunks->len[c]));
            while (i + n < steps.size() && n < (size_t)ra::kDqsMaxChunks) {
                const int64_t b = ra::ds_bytes(q->B, q->H, q->S, chunks->len[steps[i + n].c]);
                if (used + b > ds_room) break;
                used += (int64_t)round256((size_t)b);
                ++n;
            }
            if (n > 1) {
                ra::KeyMask kms[ra::kDqsMaxChunks];
                ra::DqsChunk more[ra::kDqsMaxChunks - 1];
                char* dsj = (char*)ds;
                for (size_t j = 0; j < n; ++j) {
                    const int cj = steps[i + j].c;
                    const int32_t st = chunks->start[cj], len = chunks->len[cj];
                    const ra_tensor kcj = seq_slice(*k, st, len), vcj = seq_slice(*v, st, len);
                    const ra_tensor dkj = seq_slice(dk_acc, st, len), dvj = seq_slice(dv_acc, st, len);
                    const ra_tensor dkoj = seq_slice(*dk, st, len), dvoj = seq_slice(*dv, st, len);
                    kms[j] = key_mask(kmask, st);
                    RA_HIP(ra::launch_bwd_dkdv_bf16(*q, kcj, vcj, *dout, *lse, delta, kms[j], scale, dkj, dvj, dsj, s,
                                                    direct_kv ? &dkoj : nullptr, direct_kv ? &dvoj : nullptr));
                    if (j > 0) more[j - 1] = ra::DqsChunk{kcj, dsj, kms[j].data ? &kms[j] : nullptr};
                    dsj += round256((size_t)ra::ds_bytes(q->B, q->H, q->S, len));
                }
                RA_HIP(ra::launch_bwd_dqs_bf16(*q, kc, ds, scale, dq_acc, s, !(direct_dq && i == 0),
                                               direct_dq && i + n == steps.size() ? dq : nullptr,
                                               kms[0].data ? &kms[0] : nullptr, more, (int)n - 1));
                i += n - 1;
                continue;
            }
        }
        for (int32_t r0 = 0; r0 < q->S; r0 += rows) {
            const int32_t n = std::min(rows, q->S - r0);
            const ra_tensor qs = seq_slice(*q, r0, n), dos = seq_slice(*dout, r0, n), dqs = seq_slice(dq_acc, r0, n);
            const ra_lse ls = rows_slice(*lse, r0, n), dls = rows_slice(delta, r0, n);
            const ra_tensor dqo = seq_slice(*dq, r0, n);
            RA_HIP(ra::launch_bwd_dkdv_bf16(qs, kc, vc, dos, ls, dls, km, scale, dkc, dvc, ds, s,
                                            direct_kv ? &dko : nullptr, direct_kv ? &dvo : nullptr));
            RA_HIP(ra::launch_bwd_dqs_bf16(qs, kc, ds, scale, dqs, s, !(direct_dq && i == 0),
                                           direct_dq && i + 1 == steps.size() ? &dqo : nullptr,
                                           km.data ? &km : nullptr));
        }
    }
    if (dq->dtype == RA_BF16 && !direct_dq) RA_HIP(ra::launch_cast_f32_to_bf16(dq_acc, *dq, s));
    if (dk->dtype == RA_BF16 && !direct_kv) RA_HIP(ra::launch_cast_f32_to_bf16(dk_acc, *dk, s));
    if (dv->dtype == RA_BF16 && !direct_kv) RA_HIP(ra::launch_cast_f32_to_bf16(dv_acc, *dv, s));
    return ok();
}

ra_status ra_ring_bwd(const ra_tensor* q, const ra_tensor* k, const ra_tensor* v, const ra_tensor* out,
                      const ra_tensor* dout, const ra_lse* lse, const ra_chunks* chunks, float scale, ra_tensor* dq,
                      ra_tensor* dk, ra_tensor* dv, void* ws, size_t ws_bytes, void* stream) {
    return ra_ring_bwd_masked(q, k, v, out, dout, lse, nullptr, chunks, scale, dq, dk, dv, ws, ws_bytes, stream);
}

ra_status ra_seq_head_permute(const ra_tensor* in, int32_t n_in, ra_tensor* out, int32_t n_out, int32_t dir,
                              void* stream) {
    if (dir != 0 && dir != 1) return fail(RA_E_ARG, "dir must be 0 (seq->head) or 1 (head->seq)");
    if (!in || !out) return fail(RA_E_ARG, "in/out arrays must not be NULL");
    if (n_in < 1 || n_in > ra::kMaxRanks || n_out != n_in)
        return fail(RA_E_ARG, "need 1 <= R <= %d ranks and as many outputs as inputs (got %d, %d)", ra::kMaxRanks, n_in,
                    n_out);
    const int R = n_in;
    for (int i = 0; i < R; ++i) {
        char nm[32];
        snprintf(nm, sizeof nm, "in[%d]", i);
        RA_TRY(check_tensor(&in[i], nm, true));
        snprintf(nm, sizeof nm, "out[%d]", i);
        RA_TRY(check_tensor(&out[i], nm, true));
        if (in[i].dtype != in[0].dtype || out[i].dtype != in[0].dtype)
            return fail(RA_E_DTYPE, "all exchange tensors must share one dtype");
        if (in[i].B != in[0].B || out[i].B != in[0].B || in[i].D != in[0].D || out[i].D != in[0].D)
            return fail(RA_E_SHAPE, "batch and head dim must agree across exchange tensors");
    }
    ra::PermuteTable tab;
    memset(&tab, 0, sizeof tab);
    tab.n_in = R;
    tab.n_out = R;
    tab.dir = dir;
    tab.elem_bytes = (int32_t)esize(in[0].dtype);
    // seq-side tensors (shards, all heads) and head-side tensors (head groups, whole sequence)
    const ra_tensor* seqside = dir == 0 ? in : out;
    const ra_tensor* headside = dir == 0 ? out : in;
    const int32_t H = seqside[0].H;
    const int32_t S = headside[0].S;
    tab.off[0] = 0;
    tab.hoff[0] = 0;
    for (int i = 0; i < R; ++i) {
        if (seqside[i].H != H) return fail(RA_E_SHAPE, "every sequence shard must hold all H=%d heads", H);
        if (headside[i].S != S) return fail(RA_E_SHAPE, "every head group must hold the whole sequence S=%d", S);
        tab.off[i + 1] = tab.off[i] + seqside[i].S;
        tab.hoff[i + 1] = tab.hoff[i] + headside[i].H;
    }
    if (tab.off[R] != S) return fail(RA_E_SHAPE, "shard lengths sum to %d, head groups hold S=%d", tab.off[R], S);
    if (tab.hoff[R] != H) return fail(RA_E_SHAPE, "head groups sum to %d heads, shards hold H=%d", tab.hoff[R], H);
    for (int i = 0; i < R; ++i)
        for (int j = 0; j < R; ++j) {
            uintptr_t a0, a1, b0, b1;
            byte_range(in[i], a0, a1);
            byte_range(out[j], b0, b1);
            if (a0 < b1 && b0 < a1) return fail(RA_E_ARG, "in[%d] and out[%d] overlap in memory", i, j);
        }
    for (int i = 0; i < R; ++i) {
        tab.in[i] = in[i];
        tab.out[i] = out[i];
    }
    RA_HIP(ra::launch_permute(tab, (hipStream_t)stream));
    return ok();
}

ra_status ra_split_sizes(int32_t n, int32_t parts, int32_t* sizes) {
    if (!sizes) return fail(RA_E_ARG, "sizes must not be NULL");
    if (parts < 1 || n < 0) return fail(RA_E_ARG, "need parts >= 1 and n >= 0");
    const int32_t base = n / parts, extra = n % parts;
    for (int32_t i = 0; i < parts; ++i) sizes[i] = base + (i < extra ? 1 : 0);
    return ok();
}

ra_status ra_ring_order(int32_t R, int32_t rank, int32_t* order) {
    if (!order) return fail(RA_E_ARG, "order must not be NULL");
    if (R < 1 || rank < 0 || rank >= R) return fail(RA_E_ARG, "need R >= 1 and 0 <= rank < R");
    for (int32_t i = 0; i < R; ++i) order[i] = ((rank - i) % R + R) % R;
    return ok();
}

const char* ra_status_string(ra_status s) {
    switch (s) {
        case RA_OK: return "RA_OK";
        case RA_E_ARG: return "RA_E_ARG";
        case RA_E_SHAPE: return "RA_E_SHAPE";
        case RA_E_DTYPE: return "RA_E_DTYPE";
        case RA_E_ALIGN: return "RA_E_ALIGN";
        case RA_E_UNSUPPORTED: return "RA_E_UNSUPPORTED";
        case RA_E_WORKSPACE: return "RA_E_WORKSPACE";
        case RA_E_HIP: return "RA_E_HIP";
    }
    return "RA_E_UNKNOWN";
}

const char* ra_last_error(void) { return g_err.c_str(); }

const char* ra_version(void) { return "ra 0.1 (gfx950)"; }

}  // extern "C"
