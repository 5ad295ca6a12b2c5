// Driver of the host-only sanitizer build of the C ABI (see launch_stubs.cpp): calls
// every entry point on fake device addresses, through its refusal paths (each must be
// refused with the expected status before any launch) and through the launch plans of
// the chunk steps and ring sweeps over many chunk tables, masks, layouts and workspace
// sizes (every device range a planned launch would touch must lie inside the caller's
// buffers).  Built with AddressSanitizer and UndefinedBehaviorSanitizer, any memory or
// UB error in the validation and planning code aborts the run.  Exit status 0 = clean.
#include <stdint.h>

#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "ra.h"
#include "host_check.h"

namespace {

int g_fail = 0;
int g_cases = 0;

// fake device address space: buffers 4 KiB-aligned with an unregistered 64 KiB gap after each
struct Arena {
    uintptr_t next = uintptr_t(1) << 40;
    void* get(size_t n, const char* name) {
        const uintptr_t p = next;
        next += ((n + 4095) & ~size_t(4095)) + 65536;
        hostcheck::add_alloc((void*)p, n, name);
        return (void*)p;
    }
};

size_t esz(int dt) { return dt == RA_BF16 ? 2 : 4; }

ra_tensor tensor(Arena& a, int B, int S, int H, int D, int dt, const char* name, bool seq_first = false) {
    ra_tensor t;
    t.data = a.get((size_t)B * S * H * D * esz(dt), name);
    t.dtype = dt;
    t.B = B; t.S = S; t.H = H; t.D = D;
    t.sH = D;
    if (seq_first) {
        t.sB = (int64_t)H * D;
        t.sS = (int64_t)B * H * D;
    } else {
        t.sS = (int64_t)H * D;
        t.sB = (int64_t)S * H * D;
    }
    return t;
}

ra_lse rows(Arena& a, int B, int H, int S, const char* name) {
    ra_lse l;
    l.data = (float*)a.get((size_t)B * H * S * 4, name);
    l.B = B; l.H = H; l.S = S;
    l.sH = S;
    l.sB = (int64_t)H * S;
    return l;
}

ra_kmask kmask(Arena& a, int B, int S) {
    ra_kmask m;
    m.data = (const uint8_t*)a.get((size_t)B * S, "kmask");
    m.B = B; m.S = S; m.sB = S;
    return m;
}

void expect(bool ok, const std::string& what) {
    ++g_cases;
    if (!ok) {
        ++g_fail;
        fprintf(stderr, "FAIL: %s (%s)\n", what.c_str(), ra_last_error());
    }
}

// a call that must succeed: status OK, at least one launch unless `none`, no violation
void expect_ok(ra_status st, const std::string& what, bool none = false) {
    expect(st == RA_OK, what + ": status " + ra_status_string(st));
    expect(none || hostcheck::g_launches > 0, what + ": nothing launched");
    expect(hostcheck::g_violations == 0, what + ": " + hostcheck::g_first_violation);
}

// a call that must be refused with `want` before any launch
void expect_refused(ra_status st, ra_status want, const std::string& what) {
    expect(st == want, what + ": status " + ra_status_string(st) + ", want " + ra_status_string(want));
    expect(hostcheck::g_launches == 0, what + ": launched before refusing");
    expect(std::strlen(ra_last_error()) > 0, what + ": no error text");
}

struct Chunks {
    std::vector<int32_t> start, len, order;
    ra_chunks c;
    Chunks(const std::vector<int32_t>& l, const std::vector<int32_t>& o) : len(l), order(o) {
        int32_t at = 0;
        for (int32_t x : len) {
            start.push_back(at);
            at += x;
        }
        c = ra_chunks{(int32_t)len.size(), start.data(), len.data(), order.data()};
    }
};

struct Shape {
    const char* name;
    int B, Sq, Sk, Hq, Hkv, D, dt;
    std::vector<int32_t> lens, order;
    bool seq_first;
};

void ring_case(const Shape& s, bool masked, int grad_dt, int ws_kind) {
    hostcheck::reset();
    Arena a;
    const ra_tensor q = tensor(a, s.B, s.Sq, s.Hq, s.D, s.dt, "q", s.seq_first);
    const ra_tensor k = tensor(a, s.B, s.Sk, s.Hkv, s.D, s.dt, "k", s.seq_first);
    const ra_tensor v = tensor(a, s.B, s.Sk, s.Hkv, s.D, s.dt, "v", s.seq_first);
    const ra_tensor dout = tensor(a, s.B, s.Sq, s.Hq, s.D, s.dt, "dout", s.seq_first);
    ra_tensor out = tensor(a, s.B, s.Sq, s.Hq, s.D, s.dt, "out", s.seq_first);
    ra_lse lse = rows(a, s.B, s.Hq, s.Sq, "lse");
    ra_tensor dq = tensor(a, s.B, s.Sq, s.Hq, s.D, grad_dt, "dq", s.seq_first);
    ra_tensor dk = tensor(a, s.B, s.Sk, s.Hkv, s.D, grad_dt, "dk", s.seq_first);
    ra_tensor dv = tensor(a, s.B, s.Sk, s.Hkv, s.D, grad_dt, "dv", s.seq_first);
    ra_kmask m;
    if (masked) m = kmask(a, s.B, s.Sk);
    Chunks ch(s.lens, s.order);
    std::string tag = std::string(s.name) + (masked ? " masked" : "") + (grad_dt == RA_BF16 ? " bf16-grads" : " f32-grads");
    const size_t fws = ra_ring_fwd_workspace_bytes(&q, &out);
    void* fw = fws ? a.get(fws, "fwd ws") : nullptr;
    expect_ok(ra_ring_fwd_masked(&q, &k, &v, masked ? &m : nullptr, &ch.c, 0.0883883f, &out, &lse, fw, fws, nullptr),
              tag + " ring_fwd", s.Sq == 0);
    {
        hostcheck::reset();
        Arena c;
        const ra_tensor q3 = tensor(c, s.B, s.Sq, s.Hq, s.D, s.dt, "q", s.seq_first);
        const ra_tensor k3 = tensor(c, s.B, s.Sk, s.Hkv, s.D, s.dt, "k", s.seq_first);
        const ra_tensor v3 = tensor(c, s.B, s.Sk, s.Hkv, s.D, s.dt, "v", s.seq_first);
        ra_tensor o3 = tensor(c, s.B, s.Sq, s.Hq, s.D, s.dt, "out", s.seq_first);
        ra_lse l3 = rows(c, s.B, s.Hq, s.Sq, "lse");
        ra_kmask m3;
        if (masked) m3 = kmask(c, s.B, s.Sk);
        const ra_status st = ra_ring_fwd_noalloc(&q3, &k3, &v3, masked ? &m3 : nullptr, &ch.c, 0.0883883f, &o3, &l3,
                                                 nullptr);
        if (fws <= (size_t(64) << 20))
            expect_ok(st, tag + " ring_fwd_noalloc", s.Sq == 0);
        else
            expect_refused(st, RA_E_WORKSPACE, tag + " ring_fwd_noalloc past its scratch");
    }
    const size_t lo = ra_ring_bwd_workspace_min_bytes(&q, &k, &dq, &dk, &dv);
    const size_t hi = ra_ring_bwd_workspace_bytes(&q, &k, &dq, &dk, &dv);
    expect(lo <= hi, tag + ": min workspace above recommended");
    size_t ws_bytes = 0;
    switch (ws_kind) {
        case 0: ws_bytes = lo; break;
        case 1: ws_bytes = lo + 1024; break;
        case 2: ws_bytes = lo + (hi - lo) / 3; break;
        case 3: ws_bytes = hi; break;
        case 4: ws_bytes = 2 * hi + 4096; break;
        case 5: ws_bytes = lo + (size_t(2) << 30); break;
    }
    hostcheck::reset();
    // re-register this case's buffers (reset dropped them): allocate the workspace last
    Arena b;
    const ra_tensor q2 = tensor(b, s.B, s.Sq, s.Hq, s.D, s.dt, "q", s.seq_first);
    const ra_tensor k2 = tensor(b, s.B, s.Sk, s.Hkv, s.D, s.dt, "k", s.seq_first);
    const ra_tensor v2 = tensor(b, s.B, s.Sk, s.Hkv, s.D, s.dt, "v", s.seq_first);
    const ra_tensor do2 = tensor(b, s.B, s.Sq, s.Hq, s.D, s.dt, "dout", s.seq_first);
    const ra_tensor o2 = tensor(b, s.B, s.Sq, s.Hq, s.D, s.dt, "out", s.seq_first);
    const ra_lse l2 = rows(b, s.B, s.Hq, s.Sq, "lse");
    ra_tensor dq2 = tensor(b, s.B, s.Sq, s.Hq, s.D, grad_dt, "dq", s.seq_first);
    ra_tensor dk2 = tensor(b, s.B, s.Sk, s.Hkv, s.D, grad_dt, "dk", s.seq_first);
    ra_tensor dv2 = tensor(b, s.B, s.Sk, s.Hkv, s.D, grad_dt, "dv", s.seq_first);
    ra_kmask m2;
    if (masked) m2 = kmask(b, s.B, s.Sk);
    void* ws = ws_bytes ? b.get(ws_bytes, "bwd ws") : nullptr;
    expect_ok(ra_ring_bwd_masked(&q2, &k2, &v2, &o2, &do2, &l2, masked ? &m2 : nullptr, &ch.c, 0.0883883f, &dq2, &dk2,
                                 &dv2, ws, ws_bytes, nullptr),
              tag + " ring_bwd ws#" + std::to_string(ws_kind), false);
    if (ws_kind == 0 && s.Sq > 0) {
        // below the any-table size: either a plan that needs less runs cleanly, or it is
        // refused before any launch; below delta alone it is always refused
        for (size_t short_by : {size_t(256), lo}) {
            const size_t n = lo - short_by;
            hostcheck::reset();
            Arena c;
            const ra_tensor q3 = tensor(c, s.B, s.Sq, s.Hq, s.D, s.dt, "q", s.seq_first);
            const ra_tensor k3 = tensor(c, s.B, s.Sk, s.Hkv, s.D, s.dt, "k", s.seq_first);
            const ra_tensor v3 = tensor(c, s.B, s.Sk, s.Hkv, s.D, s.dt, "v", s.seq_first);
            const ra_tensor d3 = tensor(c, s.B, s.Sq, s.Hq, s.D, s.dt, "dout", s.seq_first);
            const ra_tensor o3 = tensor(c, s.B, s.Sq, s.Hq, s.D, s.dt, "out", s.seq_first);
            const ra_lse l3 = rows(c, s.B, s.Hq, s.Sq, "lse");
            ra_tensor g0 = tensor(c, s.B, s.Sq, s.Hq, s.D, grad_dt, "dq", s.seq_first);
            ra_tensor g1 = tensor(c, s.B, s.Sk, s.Hkv, s.D, grad_dt, "dk", s.seq_first);
            ra_tensor g2 = tensor(c, s.B, s.Sk, s.Hkv, s.D, grad_dt, "dv", s.seq_first);
            void* w2 = n ? c.get(n, "short ws") : nullptr;
            const ra_status st = ra_ring_bwd(&q3, &k3, &v3, &o3, &d3, &l3, &ch.c, 0.0883883f, &g0, &g1, &g2, w2, n,
                                             nullptr);
            if (st == RA_OK && short_by != lo)
                expect_ok(st, tag + " ring_bwd below the any-table size");
            else
                expect_refused(st, RA_E_WORKSPACE, tag + " ring_bwd without room for delta");
        }
    }
}

void chunk_entry_points() {
    for (int dt : {RA_BF16, RA_F32})
        for (int D : {64, 128}) {
            hostcheck::reset();
            Arena a;
            const int B = 2, Sq = 77, Sk = 201, Hq = 6, Hkv = 2;
            const ra_tensor q = tensor(a, B, Sq, Hq, D, dt, "q"), k = tensor(a, B, Sk, Hkv, D, dt, "k");
            const ra_tensor v = tensor(a, B, Sk, Hkv, D, dt, "v"), dout = tensor(a, B, Sq, Hq, D, dt, "dout");
            ra_tensor out = tensor(a, B, Sq, Hq, D, RA_F32, "out"), part = tensor(a, B, Sq, Hq, D, RA_F32, "part");
            ra_lse lse = rows(a, B, Hq, Sq, "lse"), lpart = rows(a, B, Hq, Sq, "lpart"), delta = rows(a, B, Hq, Sq, "delta");
            ra_tensor dq = tensor(a, B, Sq, Hq, D, RA_F32, "dq"), dk = tensor(a, B, Sk, Hkv, D, RA_F32, "dk");
            ra_tensor dv = tensor(a, B, Sk, Hkv, D, RA_F32, "dv");
            ra_kmask m = kmask(a, B, Sk);
            const std::string tag = std::string(dt == RA_BF16 ? "bf16" : "f32") + " D" + std::to_string(D);
            expect_ok(ra_fwd_chunk(&q, &k, &v, 0.1f, &out, &lse, 0, nullptr), tag + " fwd_chunk");
            expect_ok(ra_fwd_chunk_masked(&q, &k, &v, &m, 0.1f, &out, &lse, 1, nullptr), tag + " fwd_chunk masked merge");
            expect_ok(ra_merge_lse(&out, &lse, &part, &lpart, nullptr), tag + " merge_lse");
            expect_ok(ra_bwd_delta(&out, &dout, &delta, nullptr), tag + " bwd_delta");
            expect_ok(ra_bwd_chunk(&q, &k, &v, &dout, &lse, &delta, 0.1f, &dq, &dk, &dv, 0, nullptr), tag + " bwd_chunk");
            expect_ok(ra_bwd_chunk_masked(&q, &k, &v, &dout, &lse, &delta, &m, 0.1f, &dq, &dk, &dv, 1, nullptr),
                      tag + " bwd_chunk masked");
            expect_ok(ra_bwd_chunk_dkdv(&q, &k, &v, &dout, &lse, &delta, 0.1f, &dk, &dv, 1, nullptr), tag + " dkdv");
            expect_ok(ra_bwd_chunk_dq(&q, &k, &v, &dout, &lse, &delta, 0.1f, &dq, nullptr), tag + " dq");
            if (dt == RA_BF16) {
                const size_t n = ra_bwd_ds_bytes(&q, &k);
                void* ds = a.get(n, "ds");
                expect_ok(ra_bwd_chunk_dkdv_ds(&q, &k, &v, &dout, &lse, &delta, &m, 0.1f, &dk, &dv, 0, ds, n, nullptr),
                          tag + " dkdv_ds");
                ra_tensor dk16 = tensor(a, B, Sk, Hkv, D, RA_BF16, "dk16"), dv16 = tensor(a, B, Sk, Hkv, D, RA_BF16, "dv16");
                expect_ok(ra_bwd_chunk_dkdv_ds(&q, &k, &v, &dout, &lse, &delta, nullptr, 0.1f, &dk16, &dv16, 0, ds, n,
                                               nullptr),
                          tag + " dkdv_ds bf16 out");
                expect_ok(ra_bwd_chunk_dq_ds(&q, &k, ds, n, 0.1f, &dq, nullptr), tag + " dq_ds");
                hostcheck::reset();
                expect_refused(ra_bwd_chunk_dq_ds(&q, &k, ds, n - 4096, 0.1f, &dq, nullptr), RA_E_WORKSPACE,
                               tag + " dq_ds short buffer");
            }
        }
}

void exchange() {
    hostcheck::reset();
    Arena a;
    const int B = 2, D = 64, H = 8;
    const int32_t sl[3] = {334, 333, 333}, hc[3] = {3, 3, 2};
    ra_tensor in[3], out[3];
    for (int i = 0; i < 3; ++i) {
        in[i] = tensor(a, B, sl[i], H, D, RA_BF16, "shard", true);
        out[i] = tensor(a, B, 1000, hc[i], D, RA_BF16, "group", true);
    }
    expect_ok(ra_seq_head_permute(in, 3, out, 3, 0, nullptr), "exchange seq->head");
    expect_ok(ra_seq_head_permute(out, 3, in, 3, 1, nullptr), "exchange head->seq");
    hostcheck::reset();
    expect_refused(ra_seq_head_permute(in, 3, out, 2, 0, nullptr), RA_E_ARG, "exchange rank mismatch");
    expect_refused(ra_seq_head_permute(in, 3, in, 3, 0, nullptr), RA_E_SHAPE, "exchange bad shapes");
    expect_refused(ra_seq_head_permute(nullptr, 3, out, 3, 0, nullptr), RA_E_ARG, "exchange null");
}

void refusals() {
    Arena a;
    const ra_tensor q = tensor(a, 1, 64, 8, 64, RA_BF16, "q"), k = tensor(a, 1, 64, 2, 64, RA_BF16, "k");
    const ra_tensor v = tensor(a, 1, 64, 2, 64, RA_BF16, "v");
    ra_tensor out = tensor(a, 1, 64, 8, 64, RA_F32, "out");
    ra_lse lse = rows(a, 1, 8, 64, "lse");
    struct Case {
        const char* name;
        ra_status want;
        void (*edit)(ra_tensor&, ra_tensor&, ra_tensor&, ra_lse&, float&);
    };
    const Case cases[] = {
        {"null data", RA_E_ARG, [](ra_tensor& q, ra_tensor&, ra_tensor&, ra_lse&, float&) { q.data = nullptr; }},
        {"bad dtype", RA_E_DTYPE, [](ra_tensor& q, ra_tensor&, ra_tensor&, ra_lse&, float&) { q.dtype = 9; }},
        {"d96", RA_E_UNSUPPORTED, [](ra_tensor& q, ra_tensor& k, ra_tensor&, ra_lse&, float&) { q.D = k.D = 96; }},
        {"misaligned", RA_E_ALIGN, [](ra_tensor& q, ra_tensor&, ra_tensor&, ra_lse&, float&) { q.data = (char*)q.data + 8; }},
        {"overlap", RA_E_ARG, [](ra_tensor& q, ra_tensor&, ra_tensor&, ra_lse&, float&) { q.sS = 8; }},
        {"negative stride", RA_E_ARG, [](ra_tensor& q, ra_tensor&, ra_tensor&, ra_lse&, float&) { q.sH = -64; }},
        {"gqa", RA_E_SHAPE, [](ra_tensor& q, ra_tensor&, ra_tensor&, ra_lse&, float&) { q.H = 6; }},
        {"lse shape", RA_E_SHAPE, [](ra_tensor&, ra_tensor&, ra_tensor&, ra_lse& l, float&) { l.S = 63; }},
        {"nan scale", RA_E_ARG, [](ra_tensor&, ra_tensor&, ra_tensor&, ra_lse&, float& s) { s = __builtin_nanf(""); }},
        {"tiny scale", RA_E_ARG, [](ra_tensor&, ra_tensor&, ra_tensor&, ra_lse&, float& s) { s = 1e-35f; }},
        {"huge S", RA_E_UNSUPPORTED, [](ra_tensor& q, ra_tensor&, ra_tensor&, ra_lse& l, float&) {
             q.S = l.S = 1 << 30; q.sB = (int64_t)q.S * q.sS; l.sB = (int64_t)l.H * l.S; }},
    };
    for (const Case& c : cases) {
        ra_tensor q2 = q, k2 = k, v2 = v;
        ra_lse l2 = lse;
        float sc = 0.125f;
        c.edit(q2, k2, v2, l2, sc);
        if (c.want == RA_E_UNSUPPORTED && std::string(c.name) == "d96") v2.D = 96;
        ra_tensor o2 = out;
        o2.D = q2.D;
        o2.S = q2.S;
        o2.sS = (int64_t)o2.H * o2.D;
        o2.sB = (int64_t)o2.S * o2.sS;
        hostcheck::reset();
        hostcheck::add_alloc(q2.data, 1, "q");
        expect_refused(ra_fwd_chunk(&q2, &k2, &v2, sc, &o2, &l2, 0, nullptr), c.want, std::string("fwd_chunk ") + c.name);
    }
    // chunk tables
    const std::vector<std::pair<std::vector<int32_t>, std::vector<int32_t>>> bad = {
        {{32, 32}, {0, 0}}, {{32, 32}, {1, 2}}, {{32, 31}, {0, 1}}, {{32, 40}, {0, 1}}, {{-1, 65}, {0, 1}}};
    for (const auto& b : bad) {
        Chunks ch(b.first, b.second);
        hostcheck::reset();
        const ra_status st = ra_ring_fwd(&q, &k, &v, &ch.c, 0.125f, &out, &lse, nullptr, 0, nullptr);
        expect(st == RA_E_ARG || st == RA_E_SHAPE, "bad chunk table accepted");
        expect(hostcheck::g_launches == 0, "bad chunk table launched");
    }
    // dout whose slice spans 2^31 bytes
    {
        const int S = 40000;
        const ra_tensor q4 = tensor(a, 1, S, 4, 128, RA_BF16, "q4"), k4 = tensor(a, 1, S, 4, 128, RA_BF16, "k4");
        ra_tensor wide = q4;
        wide.sS = 65536;
        wide.sB = (int64_t)S * 65536;
        ra_lse l4 = rows(a, 1, 4, S, "l4");
        ra_tensor a32 = tensor(a, 1, S, 4, 128, RA_F32, "acc");
        hostcheck::reset();
        expect_refused(ra_bwd_chunk(&q4, &k4, &k4, &wide, &l4, &l4, 0.125f, &a32, &a32, &a32, 1, nullptr),
                       RA_E_UNSUPPORTED, "wide dout");
    }
    // helpers
    int32_t sizes[9];
    expect(ra_split_sizes(1000, 3, sizes) == RA_OK && sizes[0] == 334 && sizes[1] == 333 && sizes[2] == 333,
           "split 1000/3");
    expect(ra_split_sizes(5, 0, sizes) == RA_E_ARG, "split by 0");
    expect(ra_ring_order(8, 0, sizes) == RA_OK && sizes[1] == 7, "ring order");
    expect(ra_ring_order(8, 8, sizes) == RA_E_ARG, "ring order bad rank");
}

}  // namespace

int main() {
    expect(hostcheck::detects_out_of_range(), "the range check misses a range one byte past a buffer");
    const std::vector<Shape> shapes = {
        {"small", 2, 200, 600, 8, 2, 64, RA_BF16, {200, 200, 200}, {1, 0, 2}, false},
        {"empty chunks", 2, 77, 201, 6, 2, 128, RA_BF16, {0, 100, 101}, {0, 1, 2}, false},
        {"empty chunks 2", 2, 77, 201, 6, 2, 128, RA_BF16, {100, 0, 101}, {1, 2, 0}, false},
        {"uneven seq-first", 2, 1000, 1000, 3, 3, 64, RA_BF16, {334, 333, 333}, {0, 2, 1}, true},
        {"no queries", 2, 0, 201, 6, 2, 128, RA_BF16, {201}, {0}, false},
        {"fp32", 1, 45, 130, 4, 2, 128, RA_F32, {65, 65}, {1, 0}, false},
        {"image-DiT", 1, 4608, 4608, 24, 24, 128, RA_BF16, {1152, 1152, 1152, 1152}, {0, 3, 2, 1}, false},
        {"video shard", 1, 4096, 32768, 32, 8, 128, RA_BF16,
         {4096, 4096, 4096, 4096, 4096, 4096, 4096, 4096}, {0, 7, 6, 5, 4, 3, 2, 1}, false},
        {"video full Q", 1, 32768, 32768, 32, 8, 128, RA_BF16,
         {4096, 4096, 4096, 4096, 4096, 4096, 4096, 4096}, {0, 1, 2, 3, 4, 5, 6, 7}, false},
        {"one 32k chunk", 1, 4096, 32768, 32, 8, 128, RA_BF16, {32768}, {0}, false},
        // ragged chunks: a third of the way from the minimum to the recommended workspace holds
        // every chunk's dS for 4288 of the 8292 rows (slice by slice, ragged last slice); the
        // recommended size holds all of it (one dQ pass)
        {"slice-major ragged", 1, 8292, 2000, 2, 1, 128, RA_BF16, {700, 1000, 300}, {1, 0, 2}, false},
        {"many chunks", 1, 512, 2000, 4, 4, 64, RA_BF16, std::vector<int32_t>(20, 100),
         {0, 19, 18, 17, 16, 15, 14, 13, 12, 11, 10, 9, 8, 7, 6, 5, 4, 3, 2, 1}, false},
    };
    for (const Shape& s : shapes)
        for (bool masked : {false, true})
            for (int gdt : {RA_BF16, RA_F32})
                for (int ws = 0; ws <= 5; ++ws) {
                    if (s.dt == RA_F32 && gdt == RA_BF16) continue;
                    ring_case(s, masked, gdt, ws);
                }
    chunk_entry_points();
    exchange();
    refusals();
    printf("host ABI check: %d checks, %d failed\n", g_cases, g_fail);
    return g_fail == 0 ? 0 : 1;
}
