// Bandwidth-bound kernels of the ring path: the standalone LSE merge, the
// backward's delta, fp32 -> bf16 finalisation, zero/row fills and the
// sequence<->head exchange.  Each thread moves 16 bytes per access so that a
// wavefront touches whole 64-byte segments.
#include "ra_device.h"

namespace ra {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int64_t toff(const ra_tensor& t, int64_t b, int64_t s, int64_t h) {
    return b * t.sB + s * t.sS + h * t.sH;
}

// n / d for 32-bit n by a multiply-high with the host-computed reciprocal of d
__device__ __forceinline__ uint32_t udiv(uint32_t n, UDiv d) {
    const uint32_t t = __umulhi(d.m, n);
    return (t + ((n - t) >> d.s1)) >> d.s2;
}

// Index i of a [B, S, H, n] iteration (n fastest) -> (b, s, h, j): by the reciprocals in
// rd when the host found every index below 2^31 (rd.fast), else by 64-bit division.
struct RowDivs {
    UDiv dn, dh, ds;
    int32_t fast;
};
__device__ __forceinline__ void split_index(int64_t i, int n, int H, int S, const RowDivs& rd, int& b, int& s, int& h,
                                            int& j) {
    if (rd.fast) {
        const uint32_t e = (uint32_t)i;
        const uint32_t q1 = udiv(e, rd.dn), q2 = udiv(q1, rd.dh), q3 = udiv(q2, rd.ds);
        j = (int)(e - q1 * (uint32_t)n);
        h = (int)(q1 - q2 * (uint32_t)H);
        s = (int)(q2 - q3 * (uint32_t)S);
        b = (int)q3;
    } else {
        j = (int)(i % n);
        int64_t r = i / n;
        h = (int)(r % H);
        r /= H;
        s = (int)(r % S);
        b = (int)(r / S);
    }
}

// ---------------------------------------------------------------- LSE merge
// One thread per (row, 4 consecutive d).  lse = log(e^a + e^b); both -inf -> (0, -inf).
__global__ __launch_bounds__(kThreads) void merge_lse_kernel(ra_tensor oa, ra_lse la, ra_tensor ob, ra_lse lb,
                                                             int64_t nvec, RowDivs rd) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= nvec) return;
    int b, s, h, d4;
    split_index(i, oa.D / 4, oa.H, oa.S, rd, b, s, h, d4);
    float* pa_l = la.data + (int64_t)b * la.sB + (int64_t)h * la.sH + s;
    const float a = *pa_l;
    const float bb = lb.data[(int64_t)b * lb.sB + (int64_t)h * lb.sH + s];
    const float m = fmaxf(a, bb);
    float wa = 0.f, wb = 0.f, lse = -INFINITY;
    if (m != -INFINITY) {
        const float ea = expf(a - m), eb = expf(bb - m);
        const float sum = ea + eb;
        lse = m + logf(sum);
        wa = ea / sum;
        wb = eb / sum;
    }
    f32x4_t* pa = (f32x4_t*)((float*)oa.data + toff(oa, b, s, h)) + d4;
    const f32x4_t* pb = (const f32x4_t*)((const float*)ob.data + toff(ob, b, s, h)) + d4;
    const f32x4_t va = *pa, vb = *pb;
    f32x4_t r4;
    for (int j = 0; j < 4; ++j) r4[j] = (wa == 0.f ? 0.f : wa * va[j]) + (wb == 0.f ? 0.f : wb * vb[j]);
    *pa = r4;
    // The D/4 threads of a row sit in one wavefront (64 % (D/4) == 0 and blocks start at
    // multiples of 256), so every lane's load of lse_acc above precedes this single store.
    if (d4 == 0) *pa_l = lse;
}

// ---------------------------------------------------------------- delta = rowsum(dO * O)
template <typename TO, typename TD>
__device__ __forceinline__ float dot8(const void* po, const void* pd);

template <>
__device__ __forceinline__ float dot8<float, float>(const void* po, const void* pd) {
    const f32x4_t* o = (const f32x4_t*)po;
    const f32x4_t* d = (const f32x4_t*)pd;
    float s = 0.f;
    for (int k = 0; k < 2; ++k)
        for (int j = 0; j < 4; ++j) s += o[k][j] * d[k][j];
    return s;
}
template <>
__device__ __forceinline__ float dot8<uint16_t, uint16_t>(const void* po, const void* pd) {
    const u32x4_t o = *(const u32x4_t*)po, d = *(const u32x4_t*)pd;
    float s = 0.f;
    for (int j = 0; j < 4; ++j) s += bf16_lo(o[j]) * bf16_lo(d[j]) + bf16_hi(o[j]) * bf16_hi(d[j]);
    return s;
}
template <>
__device__ __forceinline__ float dot8<float, uint16_t>(const void* po, const void* pd) {
    const f32x4_t* o = (const f32x4_t*)po;
    const u32x4_t d = *(const u32x4_t*)pd;
    float s = 0.f;
    for (int j = 0; j < 4; ++j) {
        const f32x4_t ov = o[j / 2];
        s += ov[2 * (j % 2)] * bf16_lo(d[j]) + ov[2 * (j % 2) + 1] * bf16_hi(d[j]);
    }
    return s;
}

// D/8 lanes per row, 8 elements each, reduced with lane shuffles.
template <typename TO, typename TD>
__global__ __launch_bounds__(kThreads) void bwd_delta_kernel(ra_tensor o, ra_tensor dout, ra_lse delta, int64_t nrows,
                                                             RowDivs rd) {
    const int L = o.D / 8;  // lanes per row: 8 or 16
    const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t row = gid >> __builtin_ctz(L);  // L = D / 8 is 8 or 16
    float s = 0.f;
    int b = 0, h = 0, sq = 0, part = 0;
    if (row < nrows) {
        split_index(gid, L, o.H, o.S, rd, b, sq, h, part);
        const TO* po = (const TO*)o.data + toff(o, b, sq, h) + part * 8;
        const TD* pd = (const TD*)dout.data + toff(dout, b, sq, h) + part * 8;
        s = dot8<TO, TD>(po, pd);
    }
    for (int w = L / 2; w >= 1; w /= 2) s += __shfl_xor(s, w, 64);
    if (row < nrows && part == 0) delta.data[(int64_t)b * delta.sB + (int64_t)h * delta.sH + sq] = s;
}

// ---------------------------------------------------------------- fp32 -> bf16 (RNE)
__global__ __launch_bounds__(kThreads) void cast_kernel(ra_tensor src, ra_tensor dst, int64_t nvec) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= nvec) return;
    const int D8 = src.D / 8;
    const int d8 = (int)(i % D8);
    int64_t r = i / D8;
    const int h = (int)(r % src.H); r /= src.H;
    const int s = (int)(r % src.S);
    const int b = (int)(r / src.S);
    const f32x4_t* ps = (const f32x4_t*)((const float*)src.data + toff(src, b, s, h)) + 2 * d8;
    const f32x4_t x0 = ps[0], x1 = ps[1];
    u32x4_t y = {pack_bf16x2(x0[0], x0[1]), pack_bf16x2(x0[2], x0[3]), pack_bf16x2(x1[0], x1[1]),
                 pack_bf16x2(x1[2], x1[3])};
    *((u32x4_t*)((uint16_t*)dst.data + toff(dst, b, s, h)) + d8) = y;
}

__global__ __launch_bounds__(kThreads) void zero_kernel(ra_tensor t, int64_t nvec) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= nvec) return;
    const int D4 = t.D / 4;
    const int d4 = (int)(i % D4);
    int64_t r = i / D4;
    const int h = (int)(r % t.H); r /= t.H;
    const int s = (int)(r % t.S);
    const int b = (int)(r / t.S);
    f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    *((f32x4_t*)((float*)t.data + toff(t, b, s, h)) + d4) = z;
}

__global__ __launch_bounds__(kThreads) void fill_rows_kernel(ra_lse t, float value, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    const int s = (int)(i % t.S);
    const int64_t r = i / t.S;
    const int h = (int)(r % t.H);
    const int b = (int)(r / t.H);
    t.data[(int64_t)b * t.sB + (int64_t)h * t.sH + s] = value;
}

// ---------------------------------------------------------------- sequence <-> head exchange
// Grid (blocks, n_out): one output tensor per blockIdx.y; each thread copies one
// 16-byte vector of a row.  The source rank is found from the offset tables.
__global__ __launch_bounds__(kThreads) void permute_kernel(PermuteTable tab) {
    const int r = blockIdx.y;
    const ra_tensor& o = tab.out[r];
    const int V = o.D * tab.elem_bytes / 16;  // vectors per (b, s, h) row
    const int64_t nvec = (int64_t)o.B * o.S * o.H * V;
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= nvec) return;
    const int v = (int)(i % V);
    int64_t rr = i / V;
    const int h = (int)(rr % o.H); rr /= o.H;
    const int s = (int)(rr % o.S);
    const int b = (int)(rr / o.S);
    const char* src;
    if (tab.dir == 0) {
        // output r = head group r over the whole sequence; row s comes from the shard holding it
        int i_src = 0;
        while (i_src + 1 < tab.n_in && s >= tab.off[i_src + 1]) ++i_src;
        const ra_tensor& x = tab.in[i_src];
        src = (const char*)x.data + toff(x, b, s - tab.off[i_src], tab.hoff[r] + h) * tab.elem_bytes;
    } else {
        // output r = sequence shard r with all heads; head h comes from the group holding it
        int g = 0;
        while (g + 1 < tab.n_in && h >= tab.hoff[g + 1]) ++g;
        const ra_tensor& x = tab.in[g];
        src = (const char*)x.data + toff(x, b, tab.off[r] + s, h - tab.hoff[g]) * tab.elem_bytes;
    }
    char* dst = (char*)o.data + toff(o, b, s, h) * tab.elem_bytes;
    ((u32x4_t*)dst)[v] = ((const u32x4_t*)src)[v];
}

// The same exchange for outputs of fewer than 2^31 vectors, split into the (output r,
// input z) sub-copies (blockIdx.y, blockIdx.z): each is a box of B x L rows x Hs heads x V
// vectors copied between fixed row and head offsets, so a block needs no search for its
// source, and a vector's (b, row, head, vector) comes from three multiply-high divisions
// instead of integer divisions.  Each thread moves four vectors, kThreads apart (every
// access of a wavefront covers 1 KiB of consecutive vectors when a row holds >= 64).
__global__ __launch_bounds__(kThreads) void permute_box_kernel(PermuteTable tab) {
    const int r = blockIdx.y, z = blockIdx.z;
    const ra_tensor& o = tab.out[r];
    const ra_tensor& x = tab.in[z];
    // dir 0 (seq -> head): rows of input shard z into output r at row off[z], heads
    //   hoff[r] .. of the input; dir 1 (head -> seq): rows off[r] .. of input group z into
    //   output r, at heads hoff[z] .. of the output
    const bool d0 = tab.dir == 0;
    const uint32_t Hs = (uint32_t)(d0 ? o.H : x.H), L = (uint32_t)(d0 ? x.S : o.S);
    const uint32_t V = (uint32_t)(o.D * tab.elem_bytes / 16);
    const UDiv dh = tab.dh[d0 ? r : z], dl = tab.dl[d0 ? z : r];
    const int64_t s_src0 = d0 ? 0 : tab.off[r], s_dst0 = d0 ? tab.off[z] : 0;
    const int64_t h_src0 = d0 ? tab.hoff[r] : 0, h_dst0 = d0 ? 0 : tab.hoff[z];
    const uint32_t nvec = (uint32_t)o.B * L * Hs * V;
    const u32x4_t* ps[4];
    u32x4_t* pd[4];
    bool ok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t e = (4 * blockIdx.x + j) * kThreads + threadIdx.x;
        ok[j] = e < nvec;
        const uint32_t q1 = udiv(e, tab.dv), v = e - q1 * V;
        const uint32_t q2 = udiv(q1, dh), h = q1 - q2 * Hs;
        const uint32_t b = udiv(q2, dl), l = q2 - b * L;
        ps[j] = (const u32x4_t*)((const char*)x.data + toff(x, b, s_src0 + l, h_src0 + h) * tab.elem_bytes) + v;
        pd[j] = (u32x4_t*)((char*)o.data + toff(o, b, s_dst0 + l, h_dst0 + h) * tab.elem_bytes) + v;
    }
    u32x4_t xv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (ok[j]) xv[j] = *ps[j];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (ok[j]) *pd[j] = xv[j];
}

inline unsigned nblocks(int64_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }

}  // namespace

static UDiv make_udiv(uint32_t d) {
    if (d == 0) return UDiv{0u, 0, 0};  // empty extent: never used
    int l = 0;
    while ((uint64_t(1) << l) < d) ++l;  // ceil(log2 d)
    const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
    return UDiv{(uint32_t)m, (uint16_t)(l < 1 ? l : 1), (uint16_t)(l > 1 ? l - 1 : 0)};
}

// reciprocals for split_index over nidx indices of a [B, S, H, n] iteration
static RowDivs row_divs(int64_t nidx, int n, int H, int S) {
    RowDivs rd{};
    rd.fast = nidx < (int64_t(1) << 31) ? 1 : 0;
    if (rd.fast) {
        rd.dn = make_udiv((uint32_t)n);
        rd.dh = make_udiv((uint32_t)H);
        rd.ds = make_udiv((uint32_t)S);
    }
    return rd;
}

hipError_t launch_merge_lse(const ra_tensor& oa, const ra_lse& la, const ra_tensor& ob, const ra_lse& lb,
                            hipStream_t s) {
    const int64_t nvec = (int64_t)oa.B * oa.S * oa.H * (oa.D / 4);
    if (nvec == 0) return hipSuccess;
    merge_lse_kernel<<<nblocks(nvec), kThreads, 0, s>>>(oa, la, ob, lb, nvec, row_divs(nvec, oa.D / 4, oa.H, oa.S));
    return hipGetLastError();
}

hipError_t launch_bwd_delta(const ra_tensor& o, const ra_tensor& dout, const ra_lse& delta, hipStream_t s) {
    const int64_t nrows = (int64_t)o.B * o.S * o.H;
    if (nrows == 0) return hipSuccess;
    const int64_t nthr = nrows * (o.D / 8);
    const unsigned g = nblocks(nthr);
    const RowDivs rd = row_divs((int64_t)g * kThreads, o.D / 8, o.H, o.S);
    if (o.dtype == RA_F32 && dout.dtype == RA_F32)
        bwd_delta_kernel<float, float><<<g, kThreads, 0, s>>>(o, dout, delta, nrows, rd);
    else if (o.dtype == RA_BF16 && dout.dtype == RA_BF16)
        bwd_delta_kernel<uint16_t, uint16_t><<<g, kThreads, 0, s>>>(o, dout, delta, nrows, rd);
    else if (o.dtype == RA_F32 && dout.dtype == RA_BF16)
        bwd_delta_kernel<float, uint16_t><<<g, kThreads, 0, s>>>(o, dout, delta, nrows, rd);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_cast_f32_to_bf16(const ra_tensor& src, const ra_tensor& dst, hipStream_t s) {
    const int64_t nvec = (int64_t)src.B * src.S * src.H * (src.D / 8);
    if (nvec == 0) return hipSuccess;
    cast_kernel<<<nblocks(nvec), kThreads, 0, s>>>(src, dst, nvec);
    return hipGetLastError();
}

hipError_t launch_zero_f32(const ra_tensor& t, hipStream_t s) {
    const int64_t nvec = (int64_t)t.B * t.S * t.H * (t.D / 4);
    if (nvec == 0) return hipSuccess;
    zero_kernel<<<nblocks(nvec), kThreads, 0, s>>>(t, nvec);
    return hipGetLastError();
}

hipError_t launch_fill_rows(const ra_lse& t, float value, hipStream_t s) {
    const int64_t n = (int64_t)t.B * t.H * t.S;
    if (n == 0) return hipSuccess;
    fill_rows_kernel<<<nblocks(n), kThreads, 0, s>>>(t, value, n);
    return hipGetLastError();
}

hipError_t launch_permute(const PermuteTable& tab_in, hipStream_t s) {
    int64_t maxvec = 0, maxbox = 0;
    bool by4 = true;
    PermuteTable tab = tab_in;
    const bool d0 = tab.dir == 0;
    for (int r = 0; r < tab.n_out; ++r) {
        const ra_tensor& o = tab.out[r];
        const int V = o.D * tab.elem_bytes / 16;
        const int64_t n = (int64_t)o.B * o.S * o.H * V;
        if (n > maxvec) maxvec = n;
        if (n >= (int64_t(1) << 31)) by4 = false;
        for (int z = 0; z < tab.n_in; ++z) {
            const ra_tensor& x = tab.in[z];
            const int64_t box = (int64_t)o.B * (d0 ? x.S : o.S) * (d0 ? o.H : x.H) * V;
            if (box > maxbox) maxbox = box;
        }
    }
    if (maxvec == 0) return hipSuccess;
    if (by4) {
        tab.dv = make_udiv((uint32_t)(tab.out[0].D * tab.elem_bytes / 16));
        for (int i = 0; i < kMaxRanks; ++i) {
            tab.dh[i] = make_udiv(i < tab.n_out ? (uint32_t)(d0 ? tab.out[i].H : tab.in[i].H) : 0u);
            tab.dl[i] = make_udiv(i < tab.n_out ? (uint32_t)(d0 ? tab.in[i].S : tab.out[i].S) : 0u);
        }
        permute_box_kernel<<<dim3((unsigned)((maxbox + 4 * kThreads - 1) / (4 * kThreads)), tab.n_out, tab.n_in),
                             kThreads, 0, s>>>(tab);
    } else {
        permute_kernel<<<dim3(nblocks(maxvec), tab.n_out), kThreads, 0, s>>>(tab);
    }
    return hipGetLastError();
}

}  // namespace ra
