// Host-only stand-ins for the kernel launchers of the ring-attention library, for
// building the C-ABI layer (argument validation, chunk tables, workspace carving, the
// launch plans of the ring sweeps) without a GPU, under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Nothing is launched.  Each stand-in records the launch
// and checks that every device byte range the kernel would touch lies inside one
// buffer the driver registered (the caller's tensors and workspace): a plan that
// carves past the end of a workspace or slices a tensor past its end is reported as a
// violation.
#include <stdint.h>

#include <cstdio>
#include <string>
#include <vector>

#include "ra_internal.h"
#include "host_check.h"

namespace hostcheck {

namespace {
struct Range {
    uintptr_t lo, hi;
    std::string name;
};
std::vector<Range> g_allocs;
}  // namespace

int g_launches = 0;
int g_violations = 0;
std::string g_first_violation;

void reset() {
    g_allocs.clear();
    g_launches = 0;
    g_violations = 0;
    g_first_violation.clear();
}

void add_alloc(const void* p, size_t n, const char* name) {
    g_allocs.push_back({(uintptr_t)p, (uintptr_t)p + n, name});
}

static void need(uintptr_t lo, uintptr_t hi, const char* what) {
    if (hi <= lo) return;
    for (const Range& a : g_allocs)
        if (lo >= a.lo && hi <= a.hi) return;
    if (g_violations++ == 0) {
        char buf[256];
        snprintf(buf, sizeof buf, "%s: bytes [%#llx, %#llx) lie in no registered buffer", what, (unsigned long long)lo,
                 (unsigned long long)hi);
        g_first_violation = buf;
    }
}

static size_t esize(int32_t dt) { return dt == RA_BF16 ? 2 : 4; }

static void need_tensor(const ra_tensor& t, const char* what) {
    if ((int64_t)t.B * t.S * t.H * t.D == 0) return;
    const int64_t last = (int64_t)(t.B - 1) * t.sB + (int64_t)(t.S - 1) * t.sS + (int64_t)(t.H - 1) * t.sH + t.D;
    need((uintptr_t)t.data, (uintptr_t)t.data + (uintptr_t)(last * (int64_t)esize(t.dtype)), what);
}

static void need_rows(const ra_lse& l, const char* what) {
    if ((int64_t)l.B * l.H * l.S == 0) return;
    const int64_t last = (int64_t)(l.B - 1) * l.sB + (int64_t)(l.H - 1) * l.sH + l.S;
    need((uintptr_t)l.data, (uintptr_t)l.data + (uintptr_t)(last * 4), what);
}

static void need_mask(const ra::KeyMask& m, int32_t B, int32_t S, const char* what) {
    if (!m.data || B * S == 0) return;
    need((uintptr_t)m.data, (uintptr_t)m.data + (uintptr_t)((int64_t)(B - 1) * m.sB + S), what);
}

static void need_ds(const void* ds, const ra_tensor& q, const ra_tensor& k, const char* what) {
    if (!ds) return;
    need((uintptr_t)ds, (uintptr_t)ds + (uintptr_t)ra::ds_bytes(q.B, q.H, q.S, k.S), what);
}

// The range check itself: a buffer's own bytes pass, one byte past its end does not.
bool detects_out_of_range() {
    reset();
    static char buf[256];
    add_alloc(buf, sizeof buf, "probe");
    need((uintptr_t)buf, (uintptr_t)buf + sizeof buf, "inside");
    const bool clean = g_violations == 0;
    need((uintptr_t)buf + 8, (uintptr_t)buf + sizeof buf + 1, "one past the end");
    const bool caught = g_violations == 1;
    reset();
    return clean && caught;
}

}  // namespace hostcheck

using namespace hostcheck;

const char* hipGetErrorString(hipError_t) { return "no device (host-only check build)"; }

namespace ra {

hipError_t launch_fwd_chunk_bf16(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const KeyMask& km,
                                 float, const ra_tensor& out, const ra_lse& lse, int merge, hipStream_t,
                                 const ra_tensor* out16) {
    ++g_launches;
    need_tensor(q, "fwd q");
    need_tensor(k, "fwd k");
    need_tensor(v, "fwd v");
    need_mask(km, q.B, k.S, "fwd kmask");
    if (merge || !out16) need_tensor(out, "fwd running out");
    if (out16) need_tensor(*out16, "fwd bf16 out");
    need_rows(lse, "fwd lse");
    return hipSuccess;
}

hipError_t launch_fwd_chunk_f32(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const KeyMask& km, float,
                                const ra_tensor& out, const ra_lse& lse, int, hipStream_t) {
    ++g_launches;
    need_tensor(q, "fwd32 q");
    need_tensor(k, "fwd32 k");
    need_tensor(v, "fwd32 v");
    need_mask(km, q.B, k.S, "fwd32 kmask");
    need_tensor(out, "fwd32 out");
    need_rows(lse, "fwd32 lse");
    return hipSuccess;
}

static void bwd_inputs(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const ra_tensor& dout,
                       const ra_lse& lse, const ra_lse& delta, const KeyMask& km, const char* who) {
    std::string w(who);
    need_tensor(q, (w + " q").c_str());
    need_tensor(k, (w + " k").c_str());
    need_tensor(v, (w + " v").c_str());
    need_tensor(dout, (w + " dout").c_str());
    need_rows(lse, (w + " lse").c_str());
    need_rows(delta, (w + " delta").c_str());
    need_mask(km, q.B, k.S, (w + " kmask").c_str());
}

hipError_t launch_bwd_dkdv_bf16(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const ra_tensor& dout,
                                const ra_lse& lse, const ra_lse& delta, const KeyMask& km, float,
                                const ra_tensor& dk_acc, const ra_tensor& dv_acc, void* ds, hipStream_t,
                                const ra_tensor* dk_out, const ra_tensor* dv_out) {
    ++g_launches;
    bwd_inputs(q, k, v, dout, lse, delta, km, "dkdv");
    if (dk_out && dv_out) {
        need_tensor(*dk_out, "dkdv bf16 dk");
        need_tensor(*dv_out, "dkdv bf16 dv");
    } else {
        need_tensor(dk_acc, "dkdv dk acc");
        need_tensor(dv_acc, "dkdv dv acc");
    }
    need_ds(ds, q, k, "dkdv dS store");
    return hipSuccess;
}

hipError_t launch_bwd_dqs_bf16(const ra_tensor& q, const ra_tensor& k, const void* ds, float, const ra_tensor& dq_acc,
                               hipStream_t, bool dq_read, const ra_tensor* dq_out, const KeyMask* km,
                               const DqsChunk* more, int n_more) {
    ++g_launches;
    need_tensor(k, "dQ pass k");
    need_ds(ds, q, k, "dQ pass dS");
    if (km) need_mask(*km, q.B, k.S, "dQ pass kmask");
    for (int i = 0; i < n_more; ++i) {
        need_tensor(more[i].k, "dQ pass k (more)");
        need_ds(more[i].ds, q, more[i].k, "dQ pass dS (more)");
        if (more[i].km) need_mask(*more[i].km, q.B, more[i].k.S, "dQ pass kmask (more)");
    }
    if (dq_read || !dq_out) need_tensor(dq_acc, "dQ pass dq acc");
    if (dq_out) need_tensor(*dq_out, "dQ pass bf16 dq");
    return hipSuccess;
}

hipError_t launch_bwd_dq_bf16(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const ra_tensor& dout,
                              const ra_lse& lse, const ra_lse& delta, const KeyMask& km, float, const ra_tensor& dq_acc,
                              hipStream_t) {
    ++g_launches;
    bwd_inputs(q, k, v, dout, lse, delta, km, "dq");
    need_tensor(dq_acc, "dq acc");
    return hipSuccess;
}

hipError_t launch_bwd_dkdv_f32(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const ra_tensor& dout,
                               const ra_lse& lse, const ra_lse& delta, const KeyMask& km, float,
                               const ra_tensor& dk_acc, const ra_tensor& dv_acc, hipStream_t) {
    ++g_launches;
    bwd_inputs(q, k, v, dout, lse, delta, km, "dkdv32");
    need_tensor(dk_acc, "dkdv32 dk");
    need_tensor(dv_acc, "dkdv32 dv");
    return hipSuccess;
}

hipError_t launch_bwd_dq_f32(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const ra_tensor& dout,
                             const ra_lse& lse, const ra_lse& delta, const KeyMask& km, float, const ra_tensor& dq_acc,
                             hipStream_t) {
    ++g_launches;
    bwd_inputs(q, k, v, dout, lse, delta, km, "dq32");
    need_tensor(dq_acc, "dq32 acc");
    return hipSuccess;
}

hipError_t launch_merge_lse(const ra_tensor& out_acc, const ra_lse& lse_acc, const ra_tensor& out_part,
                            const ra_lse& lse_part, hipStream_t) {
    ++g_launches;
    need_tensor(out_acc, "merge out acc");
    need_tensor(out_part, "merge out part");
    need_rows(lse_acc, "merge lse acc");
    need_rows(lse_part, "merge lse part");
    return hipSuccess;
}

hipError_t launch_bwd_delta(const ra_tensor& out, const ra_tensor& dout, const ra_lse& delta, hipStream_t) {
    ++g_launches;
    need_tensor(out, "delta out");
    need_tensor(dout, "delta dout");
    need_rows(delta, "delta");
    return hipSuccess;
}

hipError_t launch_cast_f32_to_bf16(const ra_tensor& src, const ra_tensor& dst, hipStream_t) {
    ++g_launches;
    need_tensor(src, "cast src");
    need_tensor(dst, "cast dst");
    return hipSuccess;
}

hipError_t launch_zero_f32(const ra_tensor& t, hipStream_t) {
    ++g_launches;
    need_tensor(t, "zero");
    return hipSuccess;
}

hipError_t launch_fill_rows(const ra_lse& t, float, hipStream_t) {
    ++g_launches;
    need_rows(t, "fill rows");
    return hipSuccess;
}

// the library's device scratch array, at a fake address registered as a buffer
hipError_t scratch_region(void** ptr, size_t* bytes) {
    void* const p = (void*)(uintptr_t(1) << 44);
    add_alloc(p, kNoAllocScratchBytes, "scratch");
    *ptr = p;
    *bytes = kNoAllocScratchBytes;
    return hipSuccess;
}

hipError_t launch_permute(const PermuteTable& tab, hipStream_t) {
    ++g_launches;
    for (int i = 0; i < tab.n_in; ++i) need_tensor(tab.in[i], "permute in");
    for (int i = 0; i < tab.n_out; ++i) need_tensor(tab.out[i], "permute out");
    return hipSuccess;
}

}  // namespace ra
