// bf16 chunk steps of ring attention on gfx950 matrix cores (MFMA 32x32x16 bf16,
// fp32 accumulate).
//
// Forward (one launch per ring step): a workgroup of 4 wavefronts owns 128 query
// rows of one (batch, query head); each wavefront keeps its 32 rows of Q in
// registers and sweeps the chunk's keys in LDS tiles of 64.  Scores are formed
// transposed, S^T = K Q^T, so that a lane owns one query row: the online-softmax
// state (running max m, running sum l) and the rescale of the output are
// lane-local, and the probabilities P^T come out of the MFMA already in the
// operand layout of the second product O^T += V^T P^T.  V stays row-major in LDS;
// its transposed operand is read with the gfx950 transposing LDS read.  The key
// tiles run as a software pipeline one tile deep (the scores of tile T + 1 are
// formed while P of tile T is exponentiated and P V of tile T accumulates).  The
// running max is only moved when a row's maximum grows by more than kRescale
// (base-2 units), so the output rescale is skipped on almost every tile.  The
// epilogue either writes the step's partial (normalised output, LSE) or merges it
// into the running fp32 (output, LSE) by LSE rescaling (the merge of the
// diffusers issue "Ring attention backward uses stale iteration-0 KV", table "How
// it surfaces per backend": ring needs LSE for partial-result merging); the last
// step of a bf16 sweep writes the merged output in bf16.
//
// Backward (one chunk step against that step's own K/V chunk - the point of that
// issue's "Root cause" and "Expected behavior") runs as two kernels with no atomics.
// The KV-stationary kernel owns 128 keys of the chunk for one KV head and sweeps the
// query rows of every query head of that GQA group in LDS tiles of 64; each 32-key
// group has two wavefronts in split roles (S, P, dV and dP, dS, dK) running one Q
// tile apart, and the workgroup adds its dK/dV rows with plain read-modify-writes
// (or, when the launch is the only one for the chunk, writes them in bf16).
// dQ takes one of two routes, both free of atomics (adding dQ from every key tile
// through device-scope atomics costs more on this chip than either).  Stored dS: the
// KV-stationary kernel also writes the dS it holds (bf16) to a caller buffer, and a
// streaming kernel forms dQ^T += K^T dS^T from it (5 products in all, 4 bytes per
// (row, key) through HBM).  Recompute: a Q-stationary kernel owns 128 query rows like
// the forward, recomputes S^T and dP^T per key tile and accumulates dQ^T += K^T dS^T in
// registers (7 products, no buffer).  Either way each row's dQ has a single writer.
//
// All kernels stream their tiles HBM -> LDS with buffer->LDS copies (rows past the
// end of a slice arrive as zeros, so tails need no branches), into unpadded rows with
// an XOR swizzle of 16-byte chunks, one tile ahead of use, with one barrier per tile;
// the per-tile work is unrolled into slots closed by scheduling barriers so that the
// operand reads stay ahead of the MFMAs that consume them.
#include <type_traits>

#include "ra_device.h"

#define RA_LDS __attribute__((address_space(3)))

namespace ra {
namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef RA_LDS uint16_t lds_u16;

constexpr float kRescale = 8.0f;  // lazy-rescale threshold of the running max, in log2 units
constexpr int kFwdStageB = 32 * 128;  // forward output staging per wavefront: 32 rows x one 128-byte line

// f(std::integral_constant<int, I>) for I = B .. E - 1, as straight-line code (the
// indices are compile-time constants inside f).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

struct FwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    float* out;
    float* lse;
    int64_t q_sB, q_sS, q_sH, k_sB, k_sS, k_sH, v_sB, v_sS, v_sH, o_sB, o_sS, o_sH, l_sB, l_sH;
    int B, Sq, Sk, Hq, G, n_qtiles;
    uint32_t k_bytes, v_bytes;  // bytes spanned by one (batch, kv head) slice of the chunk
    float c;                    // scale * log2(e)
    const uint8_t* km;          // key mask of the chunk (km[b * km_sB + key] != 0: key takes part), or null
    int64_t km_sB;
    uint16_t* out16;            // the sweep's last step: final bf16 output written here instead of out, or null
    int64_t o16_sB, o16_sS, o16_sH;
};

struct BwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* dout;
    const float* lse;
    const float* delta;
    float* dq;
    float* dk;
    float* dv;
    int64_t q_sB, q_sS, q_sH, k_sB, k_sS, k_sH, v_sB, v_sS, v_sH, do_sB, do_sS, do_sH;
    int64_t l_sB, l_sH, d_sB, d_sH;
    int64_t dq_sB, dq_sS, dq_sH, dk_sB, dk_sS, dk_sH, dv_sB, dv_sS, dv_sH;
    int B, Sq, Sk, Hq, G, n_tiles;  // tiles along the kernel's stationary axis (keys or query rows)
    uint32_t q_bytes, do_bytes, k_bytes, v_bytes;
    float scale, c, neg_inv_scale;  // neg_inv_scale = -1 / scale
    const uint8_t* km;  // key mask of the chunk (km[b * km_sB + key] != 0: key takes part), or null
    int64_t km_sB;
    // dS workspace (bf16): one 4 KiB block per (batch, query head, 32-key group, 64-row
    // query tile), ds_nkg groups x ds_nqt tiles per (batch, query head); null = none
    uint16_t* ds;
    int ds_nqt, ds_nkg;
    // dQ pass over several chunks at once (one read and write of the dQ accumulator for
    // all of them): chunk j's keys (rows of the same k tensor), length, dS blocks and key
    // mask, for j < n_dqs
    int n_dqs;
    const uint16_t* dqs_k[kDqsMaxChunks];
    uint32_t dqs_kbytes[kDqsMaxChunks];
    int dqs_Sk[kDqsMaxChunks], dqs_nkg[kDqsMaxChunks];
    const uint16_t* dqs_ds[kDqsMaxChunks];
    const uint8_t* dqs_km[kDqsMaxChunks];
    // Final bf16 outputs written once instead of the fp32 accumulators (dK/dV of a chunk
    // swept in one launch; dQ of the last chunk of a sweep), or null.  dq_read = 0: the
    // dQ pass treats the fp32 accumulator as zero (first chunk of a sweep) and stores.
    uint16_t* dk16;
    uint16_t* dv16;
    uint16_t* dq16;
    int64_t dk16_sB, dk16_sS, dk16_sH, dv16_sB, dv16_sS, dv16_sH, dq16_sB, dq16_sS, dq16_sH;
    int dq_read;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16-byte buffer load; bytes at or past the resource's size read as zero.
__device__ __forceinline__ u32x4_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

__device__ __forceinline__ float bload4f(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
}

// Resource over rows [r0, ...) of a slice that spans `bytes` bytes from `base`; the
// tile offset lives in the resource (not in soffset) so that the hardware range check
// covers it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int64_t r0, int64_t row_stride_bytes,
                                                            uint32_t bytes) {
    const int64_t off = r0 * row_stride_bytes;
    return make_rsrc((const char*)base + off, off < (int64_t)bytes ? (uint32_t)(bytes - off) : 0u);
}

__device__ __forceinline__ bf16x8_t lds_b128(const lds_u16* p) {
    return __builtin_bit_cast(bf16x8_t, *(const RA_LDS u32x4_t*)p);
}

// Key-mask bits: lane l of a wavefront loads the mask byte of key n0 + l of a 64-key
// tile (bytes past the chunk read as 0, i.e. masked); a ballot turns them into one
// 64-bit word per tile.  In a 32x32 accumulator whose rows or columns are keys, register
// r of lane l holds key 8 (r / 4) + 4 (l / 32) + r % 4 of its 32-key block kb2.
__device__ __forceinline__ uint32_t load_key_byte(const uint8_t* km_b, int Sk, int n0, int lane) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(km_b, (uint32_t)Sk);
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (uint32_t)(n0 + lane), 0, 0);
}
__device__ __forceinline__ bool key_bit(uint64_t lane_bits, int kb2, int r) {
    return (lane_bits >> (32 * kb2 + 8 * (r / 4) + (r % 4))) & 1u;
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane
// 4e+a passes the address of 4 consecutive bf16 (columns c0+4a..c0+4a+3) of row r0+e;
// lane i of the group then receives rows r0..r0+3 of column c0+i.
__device__ __forceinline__ u32x2_t lds_tr(const lds_u16* p) {
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((RA_LDS s16x4_t*)p);
    return __builtin_bit_cast(u32x2_t, v);
}

inline uint32_t span_bytes(int rows, int64_t stride, int D) {
    return rows <= 0 ? 0u : (uint32_t)(((int64_t)(rows - 1) * stride + D) * 2);
}

// Row swizzle of the unpadded Q / dO / K / V tiles in LDS: 16-byte chunk c of tile row
// r lives at chunk slot c ^ swz<RC>(r) (RC = chunks per row).  Consecutive rows (the
// 16-byte row reads of an MFMA operand) and the 4 rows x 2..4 chunks of transposing
// reads then fall on distinct bank groups.
template <int RC>
__device__ __forceinline__ int swz(int r) {
    if constexpr (RC >= 16) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return ((r & 3) << 1) | ((r >> 2) & 1);
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (stride 0, `bytes` bytes from base) as four SGPR words.
__device__ __forceinline__ i32x4_t make_desc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    i32x4_t d;
    d[0] = (int)(uint32_t)a;
    d[1] = (int)((uint32_t)(a >> 32) & 0xffffu);
    d[2] = (int)bytes;
    d[3] = 0x00020000;
    return d;
}

__device__ __forceinline__ i32x4_t tile_desc(const void* base, int64_t r0, int64_t row_stride_bytes, uint32_t bytes) {
    const int64_t off = r0 * row_stride_bytes;
    return make_desc((const char*)base + off, off < (int64_t)bytes ? (uint32_t)(bytes - off) : 0u);
}

// Asynchronous copy global -> LDS of 16 bytes per lane (buffer_load_dwordx4 ... lds):
// lane l's bytes land at dst + 16 * l, dst being the same for the whole wavefront;
// bytes past the descriptor's size arrive as zeros.  Issued as inline assembly so
// that the compiler adds no wait after it: completion is awaited explicitly with
// wait_vmem() before the barrier that publishes the tile.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(i32x4_t desc, RA_LDS void* dst, uint32_t voff) {
    const uint32_t m0v = (uint32_t)(uintptr_t)dst;
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0v), "v"(voff), "s"(desc)
                 : "memory", "m0");
}
// The same copy with the non-temporal hint, for data read exactly once (it should not
// displace reused tiles from the caches).
__device__ __forceinline__ void dma16_once(i32x4_t desc, RA_LDS void* dst, uint32_t voff) {
    const uint32_t m0v = (uint32_t)(uintptr_t)dst;
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds" ::"s"(m0v), "v"(voff), "s"(desc)
                 : "memory", "m0");
}
#pragma clang diagnostic pop
// s_waitcnt vmcnt(0): this wavefront's buffer loads (incl. the LDS copies) are done.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Copy offsets for a swizzled, unpadded tile: wavefront-wide copy `ci` moves tile rows
// [ci*RPI, +RPI) (RPI = 1024 / row bytes); lane l takes row ci*RPI + l/RC and the
// 16-byte chunk (l % RC) ^ swz(row), so that it lands at its swizzled slot.
template <int D>
__device__ __forceinline__ uint32_t copy_voff(int ci, int lane, int64_t sS) {
    constexpr int RC = D / 8, RPI = 1024 / (D * 2);
    const int r = ci * RPI + lane / RC;
    const int c = (lane % RC) ^ swz<RC>(r);
    return (uint32_t)((r * sS + 8 * c) * 2);
}

// ============================================================================ forward
template <int D, bool MERGE, bool MASK>
__global__ __launch_bounds__(64 * kFwdWaves, 2) void fwd_bf16_kernel(FwdParams p) {  // 2 wavefronts per SIMD
    constexpr int KS = D / 16, DB = D / 32, BN = kFwdBlockN, BM = kFwdBlockM;
    constexpr int RC = D / 8, ROWB = D * 2, TILEB = BN * ROWB;
    constexpr int RPI = 1024 / ROWB, NI = BN / RPI / kFwdWaves;
    constexpr int NSS = 2 * KS, NPV = 4 * DB;  // S^T and P V MFMAs per tile
    static_assert(RC >= 8 && NI >= 1, "tile geometry");
    __shared__ __attribute__((aligned(1024))) char smem[4 * TILEB];   // [K0 | V0 | K1 | V1]
    RA_LDS char* const lbase = (RA_LDS char*)smem;
    // output staging of the epilogue, 4 KiB per wavefront (32 rows x 32 fp32 columns)
    __shared__ __attribute__((aligned(16))) char ostage[kFwdWaves * kFwdStageB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    const int gq = lane >> 4, l16 = lane & 15, e4 = l16 >> 2, a4 = l16 & 3;
    const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x);
    const int qt = (int)(logical % p.n_qtiles);
    const int rest = (int)(logical / p.n_qtiles);
    const int h = rest % p.Hq, b = rest / p.Hq, g = h / p.G;
    const int row = qt * BM + w * 32 + l32;
    const bool row_ok = row < p.Sq;

    bf16x8_t qreg[KS];
    {
        const uint16_t* qrow = p.q + (int64_t)b * p.q_sB + (int64_t)row * p.q_sS + (int64_t)h * p.q_sH;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qreg[ks] = row_ok ? as_bf16x8(*(const u32x4_t*)(qrow + 16 * ks + 8 * hh))
                              : as_bf16x8(u32x4_t{0u, 0u, 0u, 0u});
    }
    f32x16_t oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16_t{};
    float m = -INFINITY, l = 0.f;

    // K/V tiles stream HBM -> LDS (swizzled rows); keys past the chunk arrive as zeros
    const uint16_t* kbase = p.k + (int64_t)b * p.k_sB + (int64_t)g * p.k_sH;
    const uint16_t* vbase = p.v + (int64_t)b * p.v_sB + (int64_t)g * p.v_sH;
    uint32_t vk[NI], vv[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        vk[i] = copy_voff<D>(w * NI + i, lane, p.k_sS);
        vv[i] = copy_voff<D>(w * NI + i, lane, p.v_sS);
    }
    const uint8_t* km_b = MASK ? p.km + (int64_t)b * p.km_sB : nullptr;
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    // LDS: [K0 | V0 | K1 | V1]; K and V tile it live in buffer it & 1.  With the key mask,
    // kbyte[buf] is the mask byte of key (tile start + lane) of the K tile in that buffer.
    uint32_t kbyte[2] = {0u, 0u};
    // Every copied tile starts inside the chunk (or the chunk is empty and tile 0 has
    // offset 0), so its byte offset is below the slice's size and fits 32 bits.
    const uint32_t k_tstep = (uint32_t)(BN * p.k_sS * 2), v_tstep = (uint32_t)(BN * p.v_sS * 2);
    auto issue_k = [&](int it, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        const uint32_t off = (uint32_t)it * k_tstep;
        const i32x4_t rk = make_desc((const char*)kbase + off, p.k_bytes - off);
        RA_LDS char* kdst = lbase + (2 * buf) * TILEB;
#pragma unroll
        for (int i = 0; i < NI; ++i) dma16(rk, kdst + (w * NI + i) * 1024, vk[i]);
        if (MASK) kbyte[buf] = load_key_byte(km_b, p.Sk, it * BN, lane);
    };
    auto issue_v = [&](int it, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        const uint32_t off = (uint32_t)it * v_tstep;
        const i32x4_t rv = make_desc((const char*)vbase + off, p.v_bytes - off);
        RA_LDS char* vdst = lbase + (2 * buf + 1) * TILEB;
#pragma unroll
        for (int i = 0; i < NI; ++i) dma16(rv, vdst + (w * NI + i) * 1024, vv[i]);
    };
    // lane-constant LDS offsets: K row reads (S^T operand) and transposing V reads (V^T operand)
    const int sw_row = swz<RC>(l32);
    int ra_off[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ra_off[ks] = l32 * ROWB + 16 * ((2 * ks + hh) ^ sw_row);
    const int sw_tr = swz<RC>(4 * hh + e4), sw_tr8 = swz<RC>(4 * hh + e4 + 8);
    int tr_off[DB], tr_off8[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        tr_off[db] = (4 * hh + e4) * ROWB + 16 * ((4 * db + 2 * (gq & 1) + (a4 >> 1)) ^ sw_tr) + 8 * (a4 & 1);
        tr_off8[db] = (4 * hh + e4) * ROWB + 16 * ((4 * db + 2 * (gq & 1) + (a4 >> 1)) ^ sw_tr8) + 8 * (a4 & 1);
    }
    auto k_read = [&](const RA_LDS char* kb, int i) {  // K rows of S^T MFMA i: key block i / KS, k-step i % KS
        return lds_b128((const lds_u16*)(kb + (i / KS) * 32 * ROWB + ra_off[i % KS]));
    };
    auto v_read = [&](const RA_LDS char* vb, int j, u32x2_t (&dst)[2]) {  // V^T operand of P V MFMA j
        const int t = j / DB, db = j % DB;
        dst[0] = lds_tr((const lds_u16*)(vb + 16 * t * ROWB + tr_off[db]));
        dst[1] = lds_tr((const lds_u16*)(vb + (16 * t + 8) * ROWB + tr_off8[db]));
    };
    // Max of a tile's scores (both 32-key blocks) in log2 units, over the lane pair that
    // shares a query row.  Masked keys and keys past the chunk (`tail`: their K rows
    // read as zero) count as -inf and are set to -inf for the exponentials.
    auto tile_max = [&](f32x16_t (&sc)[2], uint32_t kby, int n0, bool tail) {
        if (MASK) {
            const uint64_t kall = __builtin_amdgcn_ballot_w64(kby != 0);
            if (kall != ~0ull) {
                const uint64_t kl = kall >> (4 * hh);
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (!key_bit(kl, kb2, r)) sc[kb2][r] = -INFINITY;
            }
        } else if (tail) {
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (n0 + kb2 * 32 + 8 * (r / 4) + 4 * hh + (r % 4) >= p.Sk) sc[kb2][r] = -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb2][r]);
        return half_max(mx) * p.c;
    };
    // Lazy move of the running max (only when some row of the wavefront grows by more
    // than kRescale): rescales l at once and returns the factor the output accumulator
    // still has to take (1 when the max stays); `moved` (uniform) tells whether it moved.
    // Branch-free: the decision is a wavefront-uniform select.
    bool moved = false;
    auto move_max = [&](float mx) {
        moved = __builtin_amdgcn_ballot_w64(mx > m + kRescale) != 0;
        const float m_new = moved ? fmaxf(m, mx) : m;
        const float alpha = moved ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;
        l *= alpha;
        m = m_new;
        return alpha;
    };
    // Exponentials of scores 2 j, 2 j + 1 of 16-key unit t (keys 16 t .. 16 t + 15), packed
    // as bf16 into the P^T operand of the P V MFMAs of that unit
    auto exp_pair = [&](const f32x16_t (&sc)[2], int t, int j, u32x4_t& pkt) {
        const float ms = MASK && m == -INFINITY ? 0.f : m;  // row without a valid key yet
        const int r = 8 * (t % 2) + 2 * j;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t / 2][r], p.c, -ms));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t / 2][r + 1], p.c, -ms));
        l += p0 + p1;
        pkt[j] = pack_bf16x2(p0, p1);
        // keep the pair in its slot: otherwise the compiler sinks the exponentials and the
        // running sum behind the (rare) output-rescale branch that follows the slots
        asm volatile("" ::"v"(pkt[j]), "v"(l));
    };
    auto s_tile = [&](const RA_LDS char* kb, f32x16_t (&sc)[2]) {  // S^T of a whole tile, not pipelined
#pragma unroll
        for (int i = 0; i < NSS; ++i) sc[i / KS] = mfma32(k_read(kb, i), qreg[i % KS], i % KS == 0 ? f32x16_t{} : sc[i / KS]);
    };
    auto pv_tile = [&](const RA_LDS char* vb, const u32x4_t (&pk)[4]) {  // O^T += V^T P^T of a whole tile
#pragma unroll
        for (int j = 0; j < NPV; ++j) {
            u32x2_t tv[2];
            v_read(vb, j, tv);
            oacc[j % DB] = mfma32(as_bf16x8(u32x4_t{tv[0][0], tv[0][1], tv[1][0], tv[1][1]}), as_bf16x8(pk[j / DB]),
                                  oacc[j % DB]);
        }
    };
    auto rescale_out = [&](float alpha) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    };

    // Software pipeline over the chunk's full key tiles: iteration T forms P of tile T
    // (its scores S(T) and its max were produced by iteration T - 1), computes the scores
    // S(T + 1) of the next tile and adds V^T P^T of tile T.  Slots [0, NSS) run the
    // S(T + 1) MFMAs with the exponentials of units 1..3 of tile T between them; slots
    // [NSS, NSS + NPV) run the P V MFMAs of tile T with the max of tile T + 1, the move
    // of the running max and the exponentials of unit 0 of tile T + 1 between them (the
    // output accumulator takes a move's factor after the last P V MFMA).  The slot
    // region has no branch, so the compiler keeps every piece in its slot; a
    // scheduling barrier closes each slot.  K tile T + 2 and V tile T + 1 are copied
    // during iteration T (one barrier per iteration).  A partial last tile runs after
    // the loop without pipelining.
    const int ntiles_all = (p.Sk + BN - 1) / BN;
    issue_k(0, B0{});
    issue_v(0, B0{});
    if (ntiles_all > 1) issue_k(1, B1{});
    // With the key mask, the sweep ends at the last tile that holds a valid key: the tiles
    // after it (right padding) would add exactly nothing.  Each wavefront scans every
    // kFwdWaves-th tile from the end, four tiles per round, and stops at its first valid
    // key; the highest hit of the workgroup's wavefronts bounds the sweep.
    int sk_eff = p.Sk;
    if constexpr (MASK) {
        RA_LDS int* const last_valid = (RA_LDS int*)ostage;  // free until the epilogue
        int last = -1;
        for (int t0 = ntiles_all - 1 - w; t0 >= 0 && last < 0; t0 -= 4 * kFwdWaves) {
            uint32_t kb4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                kb4[j] = t0 - kFwdWaves * j >= 0 ? load_key_byte(km_b, p.Sk, (t0 - kFwdWaves * j) * BN, lane) : 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (last < 0 && __builtin_amdgcn_ballot_w64(kb4[j] != 0) != 0) last = t0 - kFwdWaves * j;
        }
        if (lane == 0) last_valid[w] = last;
        __syncthreads();
        int lv = -1;
#pragma unroll
        for (int i = 0; i < kFwdWaves; ++i) lv = max(lv, last_valid[i]);
        sk_eff = min(p.Sk, (lv + 1) * BN);
    }
    const int nfull = sk_eff / BN, ntiles = (sk_eff + BN - 1) / BN;
    wait_vmem();
    __syncthreads();
    f32x16_t sc[2];   // scores of the tile whose P is being formed
    u32x4_t pk[4];    // its P^T operands
    if (nfull > 0) {
        s_tile(lbase, sc);
        const float alpha = move_max(tile_max(sc, kbyte[0], 0, false));
        (void)alpha;  // the output accumulator is still zero
#pragma unroll
        for (int j = 0; j < 4; ++j) exp_pair(sc, 0, j, pk[0]);
    }
    __syncthreads();  // K tile 0 read by everyone before its buffer takes tile 2

    constexpr int PF = 4, LT = 2;
    auto iteration = [&](const int T, auto bufc, auto nextc) {
        constexpr int cb = decltype(bufc)::value, nb = cb ^ 1;
        constexpr bool NEXT = decltype(nextc)::value;  // tile T + 1 is a full tile
        if (T + 2 < ntiles) issue_k(T + 2, bufc);
        if (T + 1 < ntiles) issue_v(T + 1, std::integral_constant<int, nb>{});
        const RA_LDS char* kb = lbase + (2 * nb) * TILEB;      // K of tile T + 1
        const RA_LDS char* vb = lbase + (2 * cb + 1) * TILEB;  // V of tile T
        f32x16_t sn[2];
        bf16x8_t stk[NSS];
        u32x2_t trv[NPV][2];
        u32x4_t pk0n;
        float alpha = 1.f;
        if constexpr (NEXT) {
#pragma unroll
            for (int i = 0; i < PF; ++i) stk[i] = k_read(kb, i);
        }
        static_for<0, NSS + NPV>([&](auto sc_) {
            constexpr int s = decltype(sc_)::value;
            // raised wave priority over the slots that mix MFMAs with softmax work: the
            // other workgroup's wavefront on the SIMD then fills the gaps with its own
            // MFMAs rather than taking the issue slots first
            if constexpr (s == 0) __builtin_amdgcn_s_setprio(1);
            if constexpr (s == NSS + 7) __builtin_amdgcn_s_setprio(0);
            if constexpr (s < NSS) {
                if constexpr (NEXT) {
                    sn[s / KS] = mfma32(stk[s], qreg[s % KS], s % KS == 0 ? f32x16_t{} : sn[s / KS]);
                    if constexpr (s + PF < NSS) stk[s + PF] = k_read(kb, s + PF);
                }
                // exponentials of units 1..3 of tile T: 12 pairs spread over the S slots
                static_for<0, 12>([&](auto uc) {
                    constexpr int u = decltype(uc)::value;
                    if constexpr (u * NSS / 12 == s) exp_pair(sc, 1 + u / 4, u % 4, pk[1 + u / 4]);
                });
            } else {
                constexpr int j = s - NSS;
                oacc[j % DB] = mfma32(as_bf16x8(u32x4_t{trv[j][0][0], trv[j][0][1], trv[j][1][0], trv[j][1][1]}),
                                      as_bf16x8(pk[j / DB]), oacc[j % DB]);
                if constexpr (NEXT) {
                    if constexpr (j == 2) alpha = move_max(tile_max(sn, kbyte[nb], (T + 1) * BN, false));
                    if constexpr (j >= 3 && j < 7) exp_pair(sn, 0, j - 3, pk0n);
                }
            }
            if constexpr (s >= NSS - LT && s - (NSS - LT) < NPV) v_read(vb, s - (NSS - LT), trv[s - (NSS - LT)]);
            __builtin_amdgcn_sched_barrier(0);
        });
        if constexpr (NEXT) {
            if (moved) rescale_out(alpha);
            sc[0] = sn[0];
            sc[1] = sn[1];
            pk[0] = pk0n;
        }
        if (T + 1 < ntiles) wait_vmem();
        __syncthreads();
    };
    {
        int T = 0;
        for (; T + 2 < nfull; T += 2) {
            iteration(T, B0{}, std::true_type{});
            iteration(T + 1, B1{}, std::true_type{});
        }
        if (T + 1 < nfull) {
            iteration(T, B0{}, std::true_type{});
            iteration(T + 1, B1{}, std::false_type{});
        } else if (T < nfull) {
            iteration(T, B0{}, std::false_type{});
        }
    }
    if (nfull < ntiles) {
        // the partial last tile (keys past the chunk read as zero and are masked)
        const int T = nfull;
        const RA_LDS char* kb = lbase + (2 * (T & 1)) * TILEB;
        const RA_LDS char* vb = lbase + (2 * (T & 1) + 1) * TILEB;
        s_tile(kb, sc);
        const float alpha = move_max(tile_max(sc, kbyte[T & 1], T * BN, true));
        if (moved) rescale_out(alpha);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) exp_pair(sc, t, j, pk[t]);
        pv_tile(vb, pk);
    }

    l = half_sum(l);
    // Epilogue.  Row r of the result is wa(r) * (running output) + wc(r) * oacc (wa = 0 when
    // the step starts the running state).  A lane holds 4-column pieces of its one row, so
    // storing straight from the accumulators would write 32 rows x 32 bytes per instruction
    // and leave lines of the row-strided output partly written in between (the counters
    // then see up to twice the output's bytes written).
    float* lp = p.lse + (int64_t)b * p.l_sB + (int64_t)h * p.l_sH + row;
    float wa = 0.f, wc = 0.f, lse_new = -INFINITY;
    bool lse_keep = false;  // the running LSE stays as it is
    if (MASK && l == 0.f) {
        // every key of the chunk masked for this row: the step's partial is the merge
        // identity (a merge keeps the running state; a first step writes 0 and LSE -inf)
        if (MERGE) {
            wa = 1.f;
            lse_keep = true;
        }
    } else {
        const float inv_l = 1.f / l;
        const float lse_c = m * kLn2 + logf(l);
        if (!MERGE) {
            wc = inv_l;
            lse_new = lse_c;
        } else {
            // both lanes of the row (l and l^32) read lse_acc before lane l writes it
            const float la = row_ok ? *lp : 0.f;
            const float mm = fmaxf(la, lse_c);
            const float ea = expf(la - mm), ec = expf(lse_c - mm);
            const float sum = ea + ec;
            wa = ea / sum;
            wc = ec / sum * inv_l;
            lse_new = mm + logf(sum);
        }
    }
    // Each wavefront passes wc * oacc through its own 4 KiB of LDS, 32 columns (one
    // 128-byte line per row) at a time, and stores whole lines: 8 rows per instruction.
    // Branch-free but for the stores, so that the loads of the running output all issue
    // up front (a row past the end reads row Sq - 1 and stores nothing).
    RA_LDS char* const ost = (RA_LDS char*)ostage + w * kFwdStageB;
    const int rsub = lane >> 3, cc = lane & 7;  // writer lane: row 8 k + rsub, 16-byte chunk cc
    const int row0 = qt * BM + w * 32;
    float* const obase = p.out + (int64_t)b * p.o_sB + (int64_t)h * p.o_sH + 4 * cc;
    // the output of the sweep's last step goes straight to the final bf16 tensor (rounded to
    // nearest even, as the cast it replaces would)
    uint16_t* const o16base = p.out16 ? p.out16 + (int64_t)b * p.o16_sB + (int64_t)h * p.o16_sH + 4 * cc : nullptr;
    float wa_r[4];  // wa of the rows this lane writes (lane r < 32 holds row r)
    f32x4_t old[MERGE ? DB : 1][4];
    if constexpr (MERGE) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            wa_r[k] = __shfl(wa, 8 * k + rsub);
            const int64_t grow = min(row0 + 8 * k + rsub, p.Sq - 1);
#pragma unroll
            for (int db = 0; db < DB; ++db) old[db][k] = *(const f32x4_t*)(obase + grow * p.o_sS + 32 * db);
        }
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        // chunk 2 g4 + hh of row l32 (columns 32 db + 8 g4 + 4 hh .. + 3), XOR-swizzled by the
        // row's low 3 bits: the 8 lanes of one 128-byte LDS access (8 rows here, 8 chunks
        // of one row when read back) hit 8 distinct chunk positions
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4_t v4 = {wc * oacc[db][4 * g4], wc * oacc[db][4 * g4 + 1], wc * oacc[db][4 * g4 + 2],
                                wc * oacc[db][4 * g4 + 3]};
            *(RA_LDS f32x4_t*)(ost + l32 * 128 + 16 * ((2 * g4 + hh) ^ (l32 & 7))) = v4;
        }
        // LDS runs one wavefront's accesses in order: a compiler barrier suffices
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        f32x4_t v4[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int rr = 8 * k + rsub;
            v4[k] = *(const RA_LDS f32x4_t*)(ost + rr * 128 + 16 * (cc ^ (rr & 7)));
        }
        asm volatile("" ::: "memory");  // the next quarter's staging stays behind these reads
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int grow = row0 + 8 * k + rsub;
            if constexpr (MERGE) {
#pragma unroll
                for (int j = 0; j < 4; ++j) v4[k][j] += wa_r[k] == 0.f ? 0.f : wa_r[k] * old[db][k][j];
            }
            if (grow < p.Sq) {
                if (o16base)
                    *(u32x2_t*)(o16base + (int64_t)grow * p.o16_sS + 32 * db) =
                        u32x2_t{pack_bf16x2(v4[k][0], v4[k][1]), pack_bf16x2(v4[k][2], v4[k][3])};
                else
                    *(f32x4_t*)(obase + (int64_t)grow * p.o_sS + 32 * db) = v4[k];
            }
        }
    }
    if (row_ok && hh == 0 && !lse_keep) *lp = lse_new;
}

// ============================================================================ backward
// --------------------------------------------------------------- dK, dV (KV-stationary)
// Workgroup = 128 keys of the chunk x one KV head; sweeps every query row of the query
// heads sharing that KV head in tiles of 64 (so it owns its dK/dV rows and adds them
// without atomics).  Each 32-key group has two wavefronts (two per SIMD) with split
// roles, pipelined one Q tile apart so that each one's softmax arithmetic overlaps the
// other's MFMAs.  Iteration t (closed by the one barrier of the iteration) runs
//   role 0: dV += P^T dO of tile t-1, S = Q K^T of tile t, then P = exp2(c (S - lse / scale))
//           (bf16 packs for its own dV, fp16 copy to LDS for role 1);
//   role 1: dS = P (dP - delta) of tile t-1 (P from LDS), dP = dO V^T of tile t, and
//           dK += dS^T Q of tile t-1.
// Q/dO tiles are triple-buffered (tile t-1 is still read while tile t+1 lands), P
// double-buffered.  LDS starts zeroed, so the step for "tile -1" adds exact zeros, and
// one extra iteration drains the last tile (its S/dP run on a finite stale buffer and
// are discarded).  No dQ here (see bwd_dq_bf16_kernel).
template <int D>
__global__ __launch_bounds__(64 * kBwdWaves * 2) void bwd_kv_bf16_kernel(BwdParams p) {
    constexpr int KS = D / 16, DB = D / 32, BN = kBwdBlockN, BM = kBwdBlockM;
    constexpr int RB = BM / 32;            // 32-row blocks per Q tile
    constexpr int RC = D / 8;              // 16-byte chunks per row
    constexpr int ROWB = D * 2;            // bytes per (unpadded) tile row
    constexpr int TILEB = BM * ROWB;       // bytes of one Q or dO tile
    constexpr int RPI = 1024 / ROWB;       // rows moved by one wavefront-wide copy
    constexpr int NW = 2 * kBwdWaves;      // wavefronts per workgroup
    constexpr int NI = BM / RPI / NW;      // copies per wavefront per tensor per tile
    constexpr int NG = 2 * RB;             // 16-row groups per Q tile
    static_assert(RC >= 8 && NI >= 1, "tile geometry");
    constexpr int SMEMB = 6 * TILEB;                                  // [Q0 | dO0 | Q1 | dO1 | Q2 | dO2]
    constexpr int STATB = 3 * 2 * BM * 4;                             // [buffer][lse*log2e | delta][row]
    constexpr int PBUFB = 2 * kBwdWaves * 2 * RB * 64 * 16;           // [buffer][group][rb, t2][lane] (8 fp16 each)
    __shared__ __attribute__((aligned(1024))) char smem[SMEMB + STATB + PBUFB];
    RA_LDS char* const lbase = (RA_LDS char*)smem;
    RA_LDS float* const stat = (RA_LDS float*)(lbase + SMEMB);
    RA_LDS u32x4_t* const pbuf = (RA_LDS u32x4_t*)(lbase + SMEMB + STATB);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = w % kBwdWaves, role = w / kBwdWaves;
    const int l32 = lane & 31, hh = lane >> 5;
    const int gq = lane >> 4, l16 = lane & 15, e4 = l16 >> 2, a4 = l16 & 3;
    const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x);
    const int kt = (int)(logical % p.n_tiles);
    const int rest = (int)(logical / p.n_tiles);
    const int Hkv = p.Hq / p.G;
    const int g = rest % Hkv, b = rest / Hkv;
    const int n0 = kt * BN;
    const int key = n0 + 32 * kg + l32;  // this lane's key (column of S/dP, row of dK/dV)
    const bool keys_partial = n0 + BN > p.Sk;
    // a key past the chunk or masked out takes no part in dQ: its stored dS is zero
    const bool ds_zap = keys_partial || p.km != nullptr;
    uint32_t ds_keep = key < p.Sk ? ~0u : 0u;
    if (p.km && load_key_byte(p.km + (int64_t)b * p.km_sB, p.Sk, n0 + 32 * kg, l32) == 0) ds_keep = 0u;
    const int ntq = (p.Sq + BM - 1) / BM;  // Q tiles per query head
    const int ntiles = ntq * p.G;          // every Q tile of every query head of the group

    // zero all of LDS (the "tile -1" step and stale reads see finite values)
    for (int i = tid; i < (SMEMB + STATB + PBUFB) / 16; i += 64 * NW) ((RA_LDS u32x4_t*)lbase)[i] = u32x4_t{0u, 0u, 0u, 0u};

    // role 0 holds its keys' K rows, role 1 their V rows (the B operand of S or dP)
    bf16x8_t kvreg[KS];
    {
        const uint16_t* base = role == 0 ? p.k + (int64_t)b * p.k_sB + (int64_t)g * p.k_sH
                                         : p.v + (int64_t)b * p.v_sB + (int64_t)g * p.v_sH;
        const int64_t sS = role == 0 ? p.k_sS : p.v_sS;
        const uint32_t nbytes = role == 0 ? p.k_bytes : p.v_bytes;
        const __amdgpu_buffer_rsrc_t r = tile_rsrc(base, 0, sS * 2, nbytes);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kvreg[ks] = as_bf16x8(bload16(r, (uint32_t)((key * sS + 16 * ks + 8 * hh) * 2), 0));
    }
    uint32_t vq[NI], vo[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        vq[i] = copy_voff<D>(w * NI + i, lane, p.q_sS);
        vo[i] = copy_voff<D>(w * NI + i, lane, p.do_sS);
    }
    // The tile statistics (lse, delta of its 64 rows) are loaded and staged in LDS by the
    // first role-1 wavefront: role 1 ends its iteration with MFMAs and waits at the barrier
    // anyway, while role 0 ends with its softmax burst (the iteration's critical path).
    const bool stat_wave = w == kBwdWaves;
    const int stat_row = tid - 64 * kBwdWaves;
    static_assert(BM == 64, "one statistics row per lane of the staging wavefront");
    float lpre = 0.f, dpre = 0.f;
    // Tiles are copied in order: tile it is Q tile it % ntq of query head g G + it / ntq,
    // tracked incrementally (no division or 64-bit product per tile): each copy's source
    // is its head's slice base plus a 32-bit offset (a slice spans < 4 GiB) that grows by
    // one tile per copy and restarts at the next head's slice.  A copied tile always
    // starts inside its slice, so the offset never exceeds the slice's size.
    const char* q_head = (const char*)(p.q + (int64_t)b * p.q_sB + (int64_t)(g * p.G) * p.q_sH);
    const char* o_head = (const char*)(p.dout + (int64_t)b * p.do_sB + (int64_t)(g * p.G) * p.do_sH);
    const char* l_head = (const char*)(p.lse + (int64_t)b * p.l_sB + (int64_t)(g * p.G) * p.l_sH);
    const char* d_head = (const char*)(p.delta + (int64_t)b * p.d_sB + (int64_t)(g * p.G) * p.d_sH);
    const uint32_t q_tstep = (uint32_t)(BM * p.q_sS * 2), o_tstep = (uint32_t)(BM * p.do_sS * 2);
    const uint32_t lrow_bytes = (uint32_t)p.Sq * 4;
    uint32_t q_off = 0, o_off = 0, l_off = 0;
    int iss_t = 0;
    auto issue = [&](int buf) {
        const i32x4_t rq = make_desc(q_head + q_off, p.q_bytes - q_off);
        const i32x4_t ro = make_desc(o_head + o_off, p.do_bytes - o_off);
        RA_LDS char* qdst = lbase + (2 * buf) * TILEB;
        RA_LDS char* odst = lbase + (2 * buf + 1) * TILEB;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            dma16(rq, qdst + (w * NI + i) * 1024, vq[i]);
            dma16(ro, odst + (w * NI + i) * 1024, vo[i]);
        }
        if (stat_wave) {
            lpre = bload4f(make_rsrc(l_head + l_off, lrow_bytes - l_off), (uint32_t)stat_row * 4, 0);
            dpre = bload4f(make_rsrc(d_head + l_off, lrow_bytes - l_off), (uint32_t)stat_row * 4, 0);
        }
        if (++iss_t == ntq) {
            iss_t = 0;
            q_head += p.q_sH * 2;
            o_head += p.do_sH * 2;
            l_head += p.l_sH * 4;
            d_head += p.d_sH * 4;
            q_off = o_off = l_off = 0;
        } else {
            q_off += q_tstep;
            o_off += o_tstep;
            l_off += BM * 4;
        }
    };
    auto commit_stats = [&](int buf) {
        if (stat_wave) {
            // role 0 starts its S accumulator at -lse / scale, role 1 its dP accumulator at
            // -delta (scale >= 2^-100 is checked on the host, so -lse / scale is finite for
            // every finite lse; the product with the reciprocal differs from the quotient by
            // at most one rounding, 2^-24 relative)
            stat[(2 * buf) * BM + stat_row] = lpre * p.neg_inv_scale;
            stat[(2 * buf + 1) * BM + stat_row] = -dpre;
        }
    };

    // dV (role 0) or dK (role 1) of this group's 32 keys
    f32x16_t acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16_t{};
    // lane-constant LDS offsets: row reads (S, dP operands) and transposing reads (dV, dK)
    // (the role's tile within a Q/dO buffer pair is folded into these: S reads Q rows and
    // dP reads dO rows; dV reads dO^T and dK reads Q^T)
    const int own_off = role == 0 ? 0 : TILEB;
    const int oth_off = role == 0 ? TILEB : 0;
    const int sw_row = swz<RC>(l32);
    int ra_off[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ra_off[ks] = own_off + l32 * ROWB + 16 * ((2 * ks + hh) ^ sw_row);
    const int sw_tr = swz<RC>(4 * hh + e4), sw_tr8 = swz<RC>(4 * hh + e4 + 8);
    int tr_off[DB], tr_off8[DB];  // transposing reads of rows r and r + 8
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        tr_off[db] = oth_off + (4 * hh + e4) * ROWB + 16 * ((4 * db + 2 * (gq & 1) + (a4 >> 1)) ^ sw_tr) + 8 * (a4 & 1);
        tr_off8[db] = oth_off + (4 * hh + e4) * ROWB + 16 * ((4 * db + 2 * (gq & 1) + (a4 >> 1)) ^ sw_tr8) + 8 * (a4 & 1);
    }

    // Iteration slots (two MFMAs each): slot s runs the S/dP MFMA of row block s / KS at
    // k-step s % KS (tile t) and the dV/dK MFMA of group grp, column block db, j = s
    // (tile t-1).  Row reads run PF slots, transposing reads LT slots ahead.
    constexpr int NSLOT = RB * KS, PF = 3, LT = 2;
    static_assert(NSLOT == NG * DB, "one S/dP and one dV/dK MFMA per slot");
    u32x4_t pk[RB][2];   // bf16 A-operands of dV (role 0: P) or dK (role 1: dS), tile t-1
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) pk[rb][0] = pk[rb][1] = u32x4_t{0u, 0u, 0u, 0u};
    f32x16_t sacc[RB];   // S (role 0) or dP (role 1)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) sacc[rb] = f32x16_t{};

    __syncthreads();  // LDS zeroed
    issue(0);
    wait_vmem();
    commit_stats(0);
    if (ntiles > 1) issue(1);
    __syncthreads();
    // dS store of tile t-1: block (head, 32-key group, tile) of this group; within a head
    // the tiles' blocks are consecutive, the next head's start ds_nkg * ds_nqt blocks on
    char* ds_head = p.ds == nullptr ? nullptr
                                    : (char*)p.ds + ((((int64_t)b * p.Hq + g * p.G) * p.ds_nkg + n0 / 32 + kg) * p.ds_nqt) * 4096;
    const int64_t ds_hstep = (int64_t)p.ds_nkg * p.ds_nqt * 4096;
    const uint32_t ds_lane = l32 * 32 + hh * 16;
    uint32_t ds_off = 0;
    int ds_t = 0;
    // iteration it uses buffer cur = it % 3 for tile t = it (tile t-1 sits in (cur + 2) % 3);
    // the body is instantiated per cur so that the LDS addresses fold into immediates
    auto iteration = [&](const int it, auto curc) {
        constexpr int cur = decltype(curc)::value;
        constexpr int prv = cur == 0 ? 2 : cur - 1, nxt = cur == 2 ? 0 : cur + 1;
        const RA_LDS char* rowb = lbase + 2 * cur * TILEB;
        const RA_LDS char* trb = lbase + 2 * prv * TILEB;
        RA_LDS u32x4_t* const pw = pbuf + ((it & 1) * kBwdWaves + kg) * (2 * RB) * 64 + lane;        // P of tile t
        const RA_LDS u32x4_t* const pr = pbuf + (((it + 1) & 1) * kBwdWaves + kg) * (2 * RB) * 64 + lane;  // P of tile t-1

        if (role == 1) {
            // dS of tile t-1 = P (dP - delta): sacc holds dP - delta (the accumulator
            // started at -delta), P comes from LDS in fp16; one mixed-precision FMA per
            // score (v_fma_mix_f32 reads either fp16 half of the packed word)
            u32x4_t ph[RB][2];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int t2 = 0; t2 < 2; ++t2) ph[rb][t2] = pr[(2 * rb + t2) * 64];
            __builtin_amdgcn_sched_barrier(0);  // all four reads in flight before the first use
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int g4 = 2 * t2 + u;
                        float dsv[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const uint32_t word = ph[rb][t2][2 * u + j / 2];
                            const float pv = (float)__builtin_bit_cast(_Float16, (uint16_t)(j % 2 ? word >> 16 : word & 0xffffu));
                            dsv[j] = __builtin_fmaf(pv, sacc[rb][4 * g4 + j], 0.f);
                        }
                        pk[rb][t2][2 * u] = pack_bf16x2(dsv[0], dsv[1]);
                        pk[rb][t2][2 * u + 1] = pack_bf16x2(dsv[2], dsv[3]);
                    }
            // a key past the chunk or masked out: its dS is zeroed (the stored dS must be
            // zero for the dQ pass; its own dK row is never written, so dK is unaffected)
            if (ds_zap) {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
                        for (int i = 0; i < 4; ++i) pk[rb][t2][i] &= ds_keep;
            }
            if (p.ds != nullptr && it > 0) {
                // dS of tile t-1 for the dQ pass: block (head, 32-key group, tile), sub-block
                // grp = 16-row group, then key row (32 B: the lane pair's two 16-byte packs).
                // Non-temporal: the stream must not push the Q/dO tiles out of L2.
                char* blk = ds_head + ds_off + ds_lane;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int t2 = 0; t2 < 2; ++t2)
                        __builtin_nontemporal_store(pk[rb][t2], (u32x4_t*)(blk + (2 * rb + t2) * 1024));
                if (++ds_t == ntq) {
                    ds_t = 0;
                    ds_head += ds_hstep;
                    ds_off = 0;
                } else {
                    ds_off += 4096;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // Accumulator starts of tile t (register 4 g4 + j = row 32 rb + 8 g4 + 4 hh + j):
        // role 0's S accumulates onto -lse / scale of its rows (so that P = exp2(c S') with
        // c = scale log2(e)), role 1's dP onto -delta
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4_t c0 = *(const RA_LDS f32x4_t*)&stat[(2 * cur + role) * BM + 32 * rb + 8 * g4 + 4 * hh];
#pragma unroll
                for (int j = 0; j < 4; ++j) sacc[rb][4 * g4 + j] = c0[j];
            }

        {
            bf16x8_t st[NSLOT];
            u32x2_t tr[NSLOT][2];
            auto row_read = [&](int s) {
                st[s] = lds_b128((const lds_u16*)(rowb + 32 * (s / KS) * ROWB + ra_off[s % KS]));
            };
            auto tr_read = [&](int j) {  // rows 16 grp .. 16 grp + 15 of tile t-1, columns 32 db ..
                const int grp = j / DB, db = j % DB, roff = 16 * grp * ROWB;
                tr[j][0] = lds_tr((const lds_u16*)(trb + roff + tr_off[db]));
                tr[j][1] = lds_tr((const lds_u16*)(trb + roff + 8 * ROWB + tr_off8[db]));
            };
#pragma unroll
            for (int i = 0; i < PF; ++i) row_read(i);
#pragma unroll
            for (int i = 0; i < LT; ++i) tr_read(i);
            // raised priority while this wavefront issues MFMAs, so that its partner on the
            // SIMD (the other role, in its softmax burst) yields the issue slots to them
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int s = 0; s < NSLOT; ++s) {
                const int rb = s / KS, ks = s % KS, grp = s / DB, db = s % DB;
                acc[db] = mfma32(as_bf16x8(pk[grp / 2][grp % 2]),
                                 as_bf16x8(u32x4_t{tr[s][0][0], tr[s][0][1], tr[s][1][0], tr[s][1][1]}), acc[db]);
                sacc[rb] = mfma32(st[s], kvreg[ks], sacc[rb]);
                if (s + PF < NSLOT) row_read(s + PF);
                if (s + LT < NSLOT) tr_read(s + LT);
                __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_s_setprio(0);
        }

        if (role == 0) {
            // P of tile t: bf16 packs for the next iteration's dV, fp16 copy for role 1
            // lane = key, register 4 g4 + j = query row 32 rb + 8 g4 + 4 hh + j
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int t2 = 0; t2 < 2; ++t2) {
                    u32x4_t ph;
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int g4 = 2 * t2 + u;
                        float pv[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) pv[j] = __builtin_amdgcn_exp2f(sacc[rb][4 * g4 + j] * p.c);
                        pk[rb][t2][2 * u] = pack_bf16x2(pv[0], pv[1]);
                        pk[rb][t2][2 * u + 1] = pack_bf16x2(pv[2], pv[3]);
                        ph[2 * u] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(pv[0], pv[1]));
                        ph[2 * u + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(pv[2], pv[3]));
                    }
                    pw[(2 * rb + t2) * 64] = ph;
                }
        }

        // tile t+1 landed (its copy was issued an iteration ago); tile t-1's buffer and
        // this iteration's P reads are done by everyone once past the barrier
        if (it + 1 < ntiles) {
            wait_vmem();
            commit_stats(nxt);
        }
        __syncthreads();
        if (it + 2 < ntiles) issue(prv);  // tile it + 2
    };
    for (int it = 0; it <= ntiles; it += 3) {
        iteration(it, std::integral_constant<int, 0>{});
        if (it + 1 <= ntiles) iteration(it + 1, std::integral_constant<int, 1>{});
        if (it + 2 <= ntiles) iteration(it + 2, std::integral_constant<int, 2>{});
    }

    // dV (role 0) or dK (role 1) rows of this group's 32 keys: lane = d column,
    // register r = key 8*(r/4) + 4*hh + r%4.  The workgroup owns these rows (all query
    // heads of the group went through it), so a plain read-modify-write adds them.
    float* const dst = role == 0 ? p.dv + (int64_t)b * p.dv_sB + (int64_t)g * p.dv_sH + (int64_t)(n0 + 32 * kg + 4 * hh) * p.dv_sS + l32
                                 : p.dk + (int64_t)b * p.dk_sB + (int64_t)g * p.dk_sH + (int64_t)(n0 + 32 * kg + 4 * hh) * p.dk_sS + l32;
    const int64_t dst_sS = role == 0 ? p.dv_sS : p.dk_sS;
    const float mul = role == 0 ? 1.f : p.scale;
    // a masked key gets no dK/dV at all: its P and dS only ever reached its own
    // accumulator rows (lane = key in S/dP), so those rows are simply not added
    uint64_t kl_own = ~0ull;
    if (p.km) {
        const uint32_t kbyte = load_key_byte(p.km + (int64_t)b * p.km_sB, p.Sk, n0 + 32 * kg, lane & 31);
        kl_own = __builtin_amdgcn_ballot_w64(kbyte != 0 && lane < 32) >> (4 * hh);
    }
    if (p.dk16 != nullptr) {
        // the launch sweeps every query row against this chunk: write the final bf16 rows
        // (masked keys: zero) instead of adding to the fp32 accumulators
        uint16_t* const dst16 = role == 0 ? p.dv16 + (int64_t)b * p.dv16_sB + (int64_t)g * p.dv16_sH + (int64_t)(n0 + 32 * kg + 4 * hh) * p.dv16_sS + l32
                                          : p.dk16 + (int64_t)b * p.dk16_sB + (int64_t)g * p.dk16_sH + (int64_t)(n0 + 32 * kg + 4 * hh) * p.dk16_sS + l32;
        const int64_t dst16_sS = role == 0 ? p.dv16_sS : p.dk16_sS;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kr = 8 * (r / 4) + (r % 4);
                if (!keys_partial || n0 + 32 * kg + 4 * hh + kr < p.Sk) {
                    const float x = key_bit(kl_own, 0, r) ? mul * acc[db][r] : 0.f;
                    dst16[(int64_t)kr * dst16_sS + 32 * db] = (uint16_t)(pack_bf16x2(x, x) & 0xffffu);
                }
            }
        return;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kr = 8 * (r / 4) + (r % 4);
            if ((!keys_partial || n0 + 32 * kg + 4 * hh + kr < p.Sk) && key_bit(kl_own, 0, r)) {
                float* const o = dst + (int64_t)kr * dst_sS + 32 * db;
                *o += mul * acc[db][r];
            }
        }
}

// --------------------------------------------------------------- dQ (Q-stationary)
// Workgroup = 128 query rows (32 per wavefront, Q and dO rows in registers) of one
// query head; sweeps the chunk's keys in tiles of 64 like the forward.  Per tile:
// S^T = K Q^T and dP^T = V dO^T (lane = query row), P^T and dS^T with the final LSE and
// delta, then dQ^T += K^T dS^T with K^T read transposed from the K tile.  Each row's
// dQ is owned by one lane pair, so the fp32 accumulator is updated without atomics.
template <int D, bool MASK>
__global__ __launch_bounds__(256, 2) void bwd_dq_bf16_kernel(BwdParams p) {
    constexpr int KS = D / 16, DB = D / 32, BN = kFwdBlockN, BM = kFwdBlockM;
    constexpr int RC = D / 8, ROWB = D * 2, TILEB = BN * ROWB;
    constexpr int RPI = 1024 / ROWB, NI = BN / RPI / 4;
    static_assert(RC >= 8 && NI >= 1, "tile geometry");
    __shared__ __attribute__((aligned(1024))) char smem[4 * TILEB];   // [K0 | V0 | K1 | V1]
    RA_LDS char* const lbase = (RA_LDS char*)smem;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    const int gq = lane >> 4, l16 = lane & 15, e4 = l16 >> 2, a4 = l16 & 3;
    const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x);
    const int qt = (int)(logical % p.n_tiles);
    const int rest = (int)(logical / p.n_tiles);
    const int h = rest % p.Hq, b = rest / p.Hq, g = h / p.G;
    const int row = qt * BM + 32 * w + l32;
    const bool row_ok = row < p.Sq;

    bf16x8_t qreg[KS], oreg[KS];
    {
        const uint16_t* qrow = p.q + (int64_t)b * p.q_sB + (int64_t)row * p.q_sS + (int64_t)h * p.q_sH;
        const uint16_t* orow = p.dout + (int64_t)b * p.do_sB + (int64_t)row * p.do_sS + (int64_t)h * p.do_sH;
        const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qreg[ks] = as_bf16x8(row_ok ? *(const u32x4_t*)(qrow + 16 * ks + 8 * hh) : z);
            oreg[ks] = as_bf16x8(row_ok ? *(const u32x4_t*)(orow + 16 * ks + 8 * hh) : z);
        }
    }
    // rows past the end get P = 0 through an infinite LSE
    const float lse2 = row_ok ? p.lse[(int64_t)b * p.l_sB + (int64_t)h * p.l_sH + row] * kLog2e : INFINITY;
    const float dl = row_ok ? p.delta[(int64_t)b * p.d_sB + (int64_t)h * p.d_sH + row] : 0.f;

    const uint16_t* kbase = p.k + (int64_t)b * p.k_sB + (int64_t)g * p.k_sH;
    const uint16_t* vbase = p.v + (int64_t)b * p.v_sB + (int64_t)g * p.v_sH;
    uint32_t vk[NI], vv[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        vk[i] = copy_voff<D>(w * NI + i, lane, p.k_sS);
        vv[i] = copy_voff<D>(w * NI + i, lane, p.v_sS);
    }
    const uint8_t* km_b = MASK ? p.km + (int64_t)b * p.km_sB : nullptr;
    uint32_t kbyte = 0;  // mask byte of key n0 + lane of the tile in flight
    auto issue = [&](int it, int buf) {
        const int r0 = it * BN;
        const i32x4_t rk = tile_desc(kbase, r0, p.k_sS * 2, p.k_bytes);
        const i32x4_t rv = tile_desc(vbase, r0, p.v_sS * 2, p.v_bytes);
        RA_LDS char* kdst = lbase + (2 * buf) * TILEB;
        RA_LDS char* vdst = lbase + (2 * buf + 1) * TILEB;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            dma16(rk, kdst + (w * NI + i) * 1024, vk[i]);
            dma16(rv, vdst + (w * NI + i) * 1024, vv[i]);
        }
        if (MASK) kbyte = load_key_byte(km_b, p.Sk, r0, lane);
    };
    const int sw_row = swz<RC>(l32);
    int ra_off[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ra_off[ks] = l32 * ROWB + 16 * ((2 * ks + hh) ^ sw_row);
    const int sw_tr = swz<RC>(4 * hh + e4), sw_tr8 = swz<RC>(4 * hh + e4 + 8);
    int tr_off[DB], tr_off8[DB];  // transposing reads of rows r and r + 8
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        tr_off[db] = (4 * hh + e4) * ROWB + 16 * ((4 * db + 2 * (gq & 1) + (a4 >> 1)) ^ sw_tr) + 8 * (a4 & 1);
        tr_off8[db] = (4 * hh + e4) * ROWB + 16 * ((4 * db + 2 * (gq & 1) + (a4 >> 1)) ^ sw_tr8) + 8 * (a4 & 1);
    }

    f32x16_t dqacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dqacc[db] = f32x16_t{};

    issue(0, 0);
    wait_vmem();
    __syncthreads();
    // One key tile is a software pipeline of slots holding two MFMAs each: slots [0, NS)
    // compute S^T and dP^T of key block kb2 = s / KS at k-step s % KS, slots [NS, NSLOT)
    // add K^T dS^T for 16 keys t and two column blocks.  Row reads run PF slots and
    // transposing reads LT slots ahead of their MFMAs, the softmax of 16 keys two slots
    // after its key block's last S/dP MFMA; a scheduling barrier closes every slot.
    //   Keys past the chunk need no mask: their K rows read as zero, so whatever P and dS
    // they get, their share of dQ = dS K is zero.  Masked keys (key mask) get dS = 0.
    constexpr int NS = 2 * KS, SPT = DB / 2, NSLOT = NS + 4 * SPT;
    constexpr int PF = 3, LT = 2;
    static_assert(DB % 2 == 0, "two column blocks per slot");
    const int ntiles = (p.Sk + BN - 1) / BN;
    for (int it = 0; it < ntiles; ++it) {
        const int buf = it & 1;
        const bool more = it + 1 < ntiles;
        const uint64_t kall = MASK ? __builtin_amdgcn_ballot_w64(kbyte != 0) : ~0ull;  // this tile's valid keys
        const uint64_t kl = kall >> (4 * hh);
        if (more) issue(it + 1, buf ^ 1);
        if (MASK && kall == 0) {  // every key of the tile masked: dS = 0, nothing to add
            if (more) wait_vmem();
            __syncthreads();
            continue;
        }
        const bool dense = kall == ~0ull;
        const RA_LDS char* kb = lbase + (2 * buf) * TILEB;
        const RA_LDS char* vb = lbase + (2 * buf + 1) * TILEB;
        f32x16_t sacc[2], dpacc[2];
        bf16x8_t stk[NS], stv[NS];
        u32x4_t dsk[4];
        u32x2_t trk[4 * SPT][2][2];

        auto row_read = [&](int i) {
            const int kb2 = i / KS, ks = i % KS;
            stk[i] = lds_b128((const lds_u16*)(kb + kb2 * 32 * ROWB + ra_off[ks]));
            stv[i] = lds_b128((const lds_u16*)(vb + kb2 * 32 * ROWB + ra_off[ks]));
        };
        auto tr_read = [&](int j) {  // K^T operands of dQ slot j: keys 16 t .. 16 t + 15
            const int t = j / SPT, db0 = 2 * (j % SPT);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                trk[j][u][0] = lds_tr((const lds_u16*)(kb + 16 * t * ROWB + tr_off[db0 + u]));
                trk[j][u][1] = lds_tr((const lds_u16*)(kb + (16 * t + 8) * ROWB + tr_off8[db0 + u]));
            }
        };
        // dS^T = P^T * (dP^T - delta) of keys 16 t .. 16 t + 15, packed as the B operand
        auto softmax = [&](int t) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 8 * (t % 2) + 2 * j;
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t / 2][r], p.c, -lse2));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t / 2][r + 1], p.c, -lse2));
                float d0 = p0 * (dpacc[t / 2][r] - dl), d1 = p1 * (dpacc[t / 2][r + 1] - dl);
                if (MASK && !dense) {
                    d0 = key_bit(kl, t / 2, r) ? d0 : 0.f;
                    d1 = key_bit(kl, t / 2, r + 1) ? d1 : 0.f;
                }
                dsk[t][j] = pack_bf16x2(d0, d1);
            }
        };

#pragma unroll
        for (int i = 0; i < PF; ++i) row_read(i);
#pragma unroll
        for (int s = 0; s < NSLOT; ++s) {
            if (s < NS) {
                const int kb2 = s / KS, ks = s % KS;
                sacc[kb2] = mfma32(stk[s], qreg[ks], ks == 0 ? f32x16_t{} : sacc[kb2]);
                dpacc[kb2] = mfma32(stv[s], oreg[ks], ks == 0 ? f32x16_t{} : dpacc[kb2]);
                if (s + PF < NS) row_read(s + PF);
            } else {
                const int j = s - NS, t = j / SPT, db0 = 2 * (j % SPT);
                const bf16x8_t bds = as_bf16x8(dsk[t]);
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    dqacc[db0 + u] = mfma32(
                        as_bf16x8(u32x4_t{trk[j][u][0][0], trk[j][u][0][1], trk[j][u][1][0], trk[j][u][1][1]}), bds,
                        dqacc[db0 + u]);
            }
#pragma unroll
            for (int j = 0; j < 4 * SPT; ++j)
                if (s == NS + j - LT) tr_read(j);
#pragma unroll
            for (int t = 0; t < 4; ++t)
                if (s == (t / 2 + 1) * KS + 1 + t % 2) softmax(t);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (more) wait_vmem();
        __syncthreads();
    }
    if (!row_ok) return;
    // dQ^T accumulator: lane = row, register r = d 32*db + 8*(r/4) + 4*hh + r%4
    float* dqrow = p.dq + (int64_t)b * p.dq_sB + (int64_t)row * p.dq_sS + (int64_t)h * p.dq_sH;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            f32x4_t* pq = (f32x4_t*)(dqrow + 32 * db + 8 * g4 + 4 * hh);
            f32x4_t v4 = *pq;
#pragma unroll
            for (int j = 0; j < 4; ++j) v4[j] += p.scale * dqacc[db][4 * g4 + j];
            *pq = v4;
        }
}

// ------------------------------------------------------- dQ from the stored dS (Q-stationary)
// dQ = scale dS K with the dS blocks the dK/dV kernel wrote, so S and dP are not formed a
// second time.  Workgroup = kDqsWaves wavefronts x one 64-row query tile each, of one query
// head; sweeps the chunk's keys in tiles of 32 (one dS block per wavefront and tile; the
// workgroup's blocks of a tile are adjacent in memory) through a ring of kDqsStages LDS
// stages, so that three tiles are in flight while one is used: the kernel is bound by
// reading dS from HBM.  dQ^T += K^T dS^T takes both operands with transposing reads (K^T
// like V^T in the forward; dS^T from the key-major blocks).  The operands' shared k index
// runs over the 16 keys of a step in the order 4 hh + (0..3), 8 + 4 hh + (0..3) for lane
// half hh, as in the forward.
//   A dS block's 16-byte chunk c = 64 grp + 2 key + hh holds 8 entries of one key (row
// of the block) and the 16-row query group grp, in the lane order of the dK/dV kernel's
// A operand: entry 8 hh + i is dS at query row 16 grp + 4 hh + (i & 3) + 8 (i >> 2) of the
// 64-row tile (the row index with bits 2 and 3 swapped).  In LDS the four-key quads of odd groups are swapped pairwise (chunk
// c ^ 8 (grp & 1)) so that the four 16-lane quarters of a transposing read cover both
// halves of the banks.
constexpr int kDqsStages = 4;

template <int D>
__global__ __launch_bounds__(64 * kDqsWaves, 1) void bwd_dqs_bf16_kernel(BwdParams p) {
    constexpr int DB = D / 32, BN = 32;
    constexpr int RC = D / 8, ROWB = D * 2, KTB = BN * ROWB;
    constexpr int KCOPIES = KTB / 1024;                        // wavefront-wide copies per K tile
    static_assert(RC >= 8 && KCOPIES >= 1 && KCOPIES <= kDqsWaves, "tile geometry");
    constexpr int STB = KTB + kDqsWaves * 4096;                // stage: [K tile | dS block of wave 0 .. 7]
    __shared__ __attribute__((aligned(1024))) char smem[kDqsStages * STB];
    RA_LDS char* const lbase = (RA_LDS char*)smem;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hh = lane >> 5, l32 = lane & 31;
    const int gq = lane >> 4, l16 = lane & 15, e4 = l16 >> 2, a4 = l16 & 3;
    const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x);
    const int qb = (int)(logical % p.n_tiles);
    const int rest = (int)(logical / p.n_tiles);
    const int h = rest % p.Hq, b = rest / p.Hq, g = h / p.G;
    const int qt = qb * kDqsWaves + w;  // this wavefront's 64-row query tile
    const bool copies_k = w < KCOPIES;   // uniform per wavefront

    // this wavefront's dS blocks (key group t, tile qt) at (t ds_nqt + qt) of the (batch,
    // head) slab, so that a workgroup's wavefronts read adjacent blocks.  A tile at or past
    // ds_nqt (rows past the end, never stored) reads another group's block or, past the
    // slab, zeros.  With a second chunk, its key tiles follow the first chunk's.
    struct Chunk {
        const char* slab;
        int64_t slab_bytes;
        const uint16_t* kbase;
        uint32_t kbytes;
    };
    auto chunk_of = [&](int j) {
        const int64_t slab_blocks = (int64_t)p.ds_nqt * p.dqs_nkg[j];
        return Chunk{(const char*)p.dqs_ds[j] + ((int64_t)b * p.Hq + h) * slab_blocks * 4096, slab_blocks * 4096,
                     p.dqs_k[j] + (int64_t)b * p.k_sB + (int64_t)g * p.k_sH, p.dqs_kbytes[j]};
    };
    uint32_t vds[4];  // copy offsets: LDS chunk 64 i + lane <- block chunk (64 i + lane) ^ 8 (i & 1)
#pragma unroll
    for (int i = 0; i < 4; ++i) vds[i] = (uint32_t)(((64 * i + lane) ^ (8 * (i & 1))) * 16);

    const uint32_t vk = copy_voff<D>(w, lane, p.k_sS);
    int ntk[kDqsMaxChunks];  // key tiles of each chunk
    // Tiles are issued in order (it = 0, 1, ...): tile it is key tile t of chunk j, tracked
    // incrementally.  Tile it goes to stage it % kDqsStages: one K copy (first KCOPIES
    // wavefronts) and the wavefront's own dS block.  A copied K tile starts inside its
    // chunk, so its byte offset is below the slice's size and fits 32 bits; the dS offset
    // can pass the slab (tiles at or past ds_nqt), where the copy reads zeros.
    int iss_j = 0, iss_t = 0;
    Chunk iss_c = chunk_of(0);
    const uint32_t k_tstep = (uint32_t)(BN * p.k_sS * 2);
    const int64_t ds_tstep = (int64_t)p.ds_nqt * 4096;
    auto ntk_of = [&](int j) {  // ntk[j] through selects (no dynamically indexed register array)
        int n = 0;
#pragma unroll
        for (int jj = 0; jj < kDqsMaxChunks; ++jj)
            if (jj == j) n = ntk[jj];
        return n;
    };
    auto issue = [&](int it) {
        while (iss_t == ntk_of(iss_j)) {  // next chunk with key tiles (only existing tiles are issued)
            iss_t = 0;
            iss_c = chunk_of(++iss_j);
        }
        RA_LDS char* st = lbase + (it % kDqsStages) * STB;
        const uint32_t koff = (uint32_t)iss_t * k_tstep;
        if (copies_k) dma16(make_desc((const char*)iss_c.kbase + koff, iss_c.kbytes - koff), st + w * 1024, vk);
        const int64_t off = iss_t * ds_tstep + (int64_t)qt * 4096;
        const i32x4_t rd = make_desc(iss_c.slab + off, off < iss_c.slab_bytes ? (uint32_t)(iss_c.slab_bytes - off) : 0u);
#pragma unroll
        for (int i = 0; i < 4; ++i) dma16_once(rd, st + KTB + w * 4096 + i * 1024, vds[i]);
        ++iss_t;
    };
    // lane-constant LDS offsets: K^T reads (as V^T in the forward) and dS^T reads
    const int sw_tr = swz<RC>(4 * hh + e4), sw_tr8 = swz<RC>(4 * hh + e4 + 8);
    int tr_off[DB], tr_off8[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        tr_off[db] = (4 * hh + e4) * ROWB + 16 * ((4 * db + 2 * (gq & 1) + (a4 >> 1)) ^ sw_tr) + 8 * (a4 & 1);
        tr_off8[db] = (4 * hh + e4) * ROWB + 16 * ((4 * db + 2 * (gq & 1) + (a4 >> 1)) ^ sw_tr8) + 8 * (a4 & 1);
    }
    // dS^T operand of query block qr (32 rows = groups 2 qr, 2 qr + 1), keys 16 t + (0..15):
    // quarter gq reads group 2 qr + (gq & 1), keys 16 t + 4 hh + e4 and 16 t + 8 + 4 hh + e4,
    // columns 4 a4 .. 4 a4 + 3
    auto ds_off = [&](int qr, int key) {
        const int grp = 2 * qr + (gq & 1);
        return grp * 1024 + ((((key >> 2) ^ (grp & 1)) * 8 + (key & 3) * 2 + (a4 >> 1)) * 16) + 8 * (a4 & 1);
    };
    int dso[2][2][2];  // [query block][key step][first / second read]
#pragma unroll
    for (int qr = 0; qr < 2; ++qr)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            dso[qr][t][0] = ds_off(qr, 16 * t + 4 * hh + e4);
            dso[qr][t][1] = ds_off(qr, 16 * t + 8 + 4 * hh + e4);
        }

    f32x16_t acc[2][DB];
#pragma unroll
    for (int qr = 0; qr < 2; ++qr)
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[qr][db] = f32x16_t{};

    // Key tiles of a chunk.  With its key mask: dS of the keys after the last valid key is
    // zero, so the tiles end at the 64-key tile that holds that key (each wavefront scans
    // every kDqsWaves-th tile from the end; the highest hit bounds the loop).  One word of
    // LDS per wavefront carries the hits, before any tile copy lands there.
    auto key_tiles = [&](const uint8_t* km, int Sk) {
        if (km == nullptr) return (Sk + BN - 1) / BN;
        const uint8_t* km_b = km + (int64_t)b * p.km_sB;
        const int nt64 = (Sk + 63) / 64;
        int last = -1;
        for (int t0 = nt64 - 1 - w; t0 >= 0 && last < 0; t0 -= 4 * kDqsWaves) {
            uint32_t kb4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                kb4[j] = t0 - kDqsWaves * j >= 0 ? load_key_byte(km_b, Sk, (t0 - kDqsWaves * j) * 64, lane) : 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (last < 0 && __builtin_amdgcn_ballot_w64(kb4[j] != 0) != 0) last = t0 - kDqsWaves * j;
        }
        RA_LDS int* const hits = (RA_LDS int*)lbase;
        if (lane == 0) hits[w] = last;
        __syncthreads();
        int lv = -1;
#pragma unroll
        for (int i = 0; i < kDqsWaves; ++i) lv = max(lv, hits[i]);
        __syncthreads();
        return (min(Sk, (lv + 1) * 64) + BN - 1) / BN;
    };
    int ntiles = 0;
#pragma unroll
    for (int j = 0; j < kDqsMaxChunks; ++j) {
        ntk[j] = j < p.n_dqs ? key_tiles(p.dqs_km[j], p.dqs_Sk[j]) : 0;
        ntiles += ntk[j];
    }
#pragma unroll
    for (int i = 0; i < kDqsStages - 1; ++i)
        if (i < ntiles) issue(i);
    for (int it = 0; it < ntiles; ++it) {
        // tile it has landed once at most the copies of the (up to two) later tiles
        // issued so far are outstanding: 4 dS copies + 1 K copy per tile and wavefront
        const int later = min(ntiles - 1 - it, kDqsStages - 2);
        if (copies_k) {
            if (later >= 2) __builtin_amdgcn_s_waitcnt(0x0F70 | 10);
            else if (later == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | 5);
            else wait_vmem();
        } else {
            if (later >= 2) __builtin_amdgcn_s_waitcnt(0x0F70 | 8);
            else if (later == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | 4);
            else wait_vmem();
        }
        // after the barrier every wavefront's part of tile it is visible and the stage of
        // tile it - 1 is free again
        __syncthreads();
        if (it + kDqsStages - 1 < ntiles) issue(it + kDqsStages - 1);
        const RA_LDS char* kb = lbase + (it % kDqsStages) * STB;
        const RA_LDS char* dsb = kb + KTB + w * 4096;
#pragma unroll
        for (int t = 0; t < 2; ++t) {  // 16 keys 16 t .. 16 t + 15 of the tile
            u32x2_t kf[DB][2], df[2][2];
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                kf[db][0] = lds_tr((const lds_u16*)(kb + 16 * t * ROWB + tr_off[db]));
                kf[db][1] = lds_tr((const lds_u16*)(kb + (16 * t + 8) * ROWB + tr_off8[db]));
            }
#pragma unroll
            for (int qr = 0; qr < 2; ++qr) {
                df[qr][0] = lds_tr((const lds_u16*)(dsb + dso[qr][t][0]));
                df[qr][1] = lds_tr((const lds_u16*)(dsb + dso[qr][t][1]));
            }
#pragma unroll
            for (int qr = 0; qr < 2; ++qr)
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    acc[qr][db] = mfma32(as_bf16x8(u32x4_t{kf[db][0][0], kf[db][0][1], kf[db][1][0], kf[db][1][1]}),
                                         as_bf16x8(u32x4_t{df[qr][0][0], df[qr][0][1], df[qr][1][0], df[qr][1][1]}),
                                         acc[qr][db]);
        }
    }
    // dQ^T accumulator of query block qr: lane = query row 32 qr + (l32 with bits 2 and 3
    // swapped) of the tile, register r = d 32 db + 8 (r / 4) + 4 hh + r % 4
    // dq_read = 0: the accumulator counts as zero; dq16: write the final bf16 rows instead
    const int rloc = (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
#pragma unroll
    for (int qr = 0; qr < 2; ++qr) {
        const int row = qt * 64 + 32 * qr + rloc;
        if (row >= p.Sq) continue;
        float* dqrow = p.dq + (int64_t)b * p.dq_sB + (int64_t)row * p.dq_sS + (int64_t)h * p.dq_sH;
        uint16_t* dq16row = p.dq16 ? p.dq16 + (int64_t)b * p.dq16_sB + (int64_t)row * p.dq16_sS + (int64_t)h * p.dq16_sH
                                   : nullptr;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                f32x4_t* pq = (f32x4_t*)(dqrow + 32 * db + 8 * g4 + 4 * hh);
                f32x4_t v4 = p.dq_read ? *pq : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 4; ++j) v4[j] += p.scale * acc[qr][db][4 * g4 + j];
                if (dq16row)
                    *(u32x2_t*)(dq16row + 32 * db + 8 * g4 + 4 * hh) = u32x2_t{pack_bf16x2(v4[0], v4[1]), pack_bf16x2(v4[2], v4[3])};
                else
                    *pq = v4;
            }
    }
}

}  // namespace

hipError_t launch_fwd_chunk_bf16(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const KeyMask& km,
                                 float scale, const ra_tensor& out, const ra_lse& lse, int merge, hipStream_t s,
                                 const ra_tensor* out16) {
    if (q.S == 0 || k.S == 0) return hipSuccess;
    FwdParams p;
    p.q = (const uint16_t*)q.data;
    p.k = (const uint16_t*)k.data;
    p.v = (const uint16_t*)v.data;
    p.out = (float*)out.data;
    p.lse = lse.data;
    p.q_sB = q.sB; p.q_sS = q.sS; p.q_sH = q.sH;
    p.k_sB = k.sB; p.k_sS = k.sS; p.k_sH = k.sH;
    p.v_sB = v.sB; p.v_sS = v.sS; p.v_sH = v.sH;
    p.o_sB = out.sB; p.o_sS = out.sS; p.o_sH = out.sH;
    p.l_sB = lse.sB; p.l_sH = lse.sH;
    p.B = q.B; p.Sq = q.S; p.Sk = k.S; p.Hq = q.H; p.G = q.H / k.H;
    p.n_qtiles = (q.S + kFwdBlockM - 1) / kFwdBlockM;
    p.k_bytes = span_bytes(k.S, k.sS, k.D);
    p.v_bytes = span_bytes(v.S, v.sS, v.D);
    p.c = scale * 1.4426950408889634f;
    const unsigned nb = (unsigned)p.n_qtiles * q.H * q.B;
    p.km = km.data;
    p.km_sB = km.sB;
    p.out16 = out16 ? (uint16_t*)out16->data : nullptr;
    p.o16_sB = out16 ? out16->sB : 0;
    p.o16_sS = out16 ? out16->sS : 0;
    p.o16_sH = out16 ? out16->sH : 0;
    const bool mk = km.data != nullptr;
    if (q.D == 64) {
        if (merge) mk ? fwd_bf16_kernel<64, true, true><<<nb, 64 * kFwdWaves, 0, s>>>(p) : fwd_bf16_kernel<64, true, false><<<nb, 64 * kFwdWaves, 0, s>>>(p);
        else mk ? fwd_bf16_kernel<64, false, true><<<nb, 64 * kFwdWaves, 0, s>>>(p) : fwd_bf16_kernel<64, false, false><<<nb, 64 * kFwdWaves, 0, s>>>(p);
    } else {
        if (merge) mk ? fwd_bf16_kernel<128, true, true><<<nb, 64 * kFwdWaves, 0, s>>>(p) : fwd_bf16_kernel<128, true, false><<<nb, 64 * kFwdWaves, 0, s>>>(p);
        else mk ? fwd_bf16_kernel<128, false, true><<<nb, 64 * kFwdWaves, 0, s>>>(p) : fwd_bf16_kernel<128, false, false><<<nb, 64 * kFwdWaves, 0, s>>>(p);
    }
    return hipGetLastError();
}

namespace {
BwdParams bwd_params(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const ra_tensor& dout,
                     const ra_lse& lse, const ra_lse& delta, float scale) {
    BwdParams p;
    p.q = (const uint16_t*)q.data;
    p.k = (const uint16_t*)k.data;
    p.v = (const uint16_t*)v.data;
    p.dout = (const uint16_t*)dout.data;
    p.lse = lse.data;
    p.delta = delta.data;
    p.dq = p.dk = p.dv = nullptr;
    p.q_sB = q.sB; p.q_sS = q.sS; p.q_sH = q.sH;
    p.k_sB = k.sB; p.k_sS = k.sS; p.k_sH = k.sH;
    p.v_sB = v.sB; p.v_sS = v.sS; p.v_sH = v.sH;
    p.do_sB = dout.sB; p.do_sS = dout.sS; p.do_sH = dout.sH;
    p.l_sB = lse.sB; p.l_sH = lse.sH;
    p.d_sB = delta.sB; p.d_sH = delta.sH;
    p.dq_sB = p.dq_sS = p.dq_sH = p.dk_sB = p.dk_sS = p.dk_sH = p.dv_sB = p.dv_sS = p.dv_sH = 0;
    p.B = q.B; p.Sq = q.S; p.Sk = k.S; p.Hq = q.H; p.G = q.H / k.H;
    p.n_tiles = 0;
    p.q_bytes = span_bytes(q.S, q.sS, q.D);
    p.do_bytes = span_bytes(dout.S, dout.sS, dout.D);
    p.k_bytes = span_bytes(k.S, k.sS, k.D);
    p.v_bytes = span_bytes(v.S, v.sS, v.D);
    p.scale = scale;
    p.c = scale * 1.4426950408889634f;
    p.neg_inv_scale = (float)(-1.0 / (double)scale);
    p.km = nullptr;
    p.km_sB = 0;
    p.ds = nullptr;
    p.n_dqs = 0;
    p.ds_nqt = p.ds_nkg = 0;
    p.dk16 = p.dv16 = p.dq16 = nullptr;
    p.dk16_sB = p.dk16_sS = p.dk16_sH = p.dv16_sB = p.dv16_sS = p.dv16_sH = p.dq16_sB = p.dq16_sS = p.dq16_sH = 0;
    p.dq_read = 1;
    return p;
}
}  // namespace

hipError_t launch_bwd_dkdv_bf16(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const ra_tensor& dout,
                                const ra_lse& lse, const ra_lse& delta, const KeyMask& km, float scale,
                                const ra_tensor& dk_acc, const ra_tensor& dv_acc, void* ds, hipStream_t s,
                                const ra_tensor* dk_out, const ra_tensor* dv_out) {
    if (q.S == 0 || k.S == 0) return hipSuccess;
    BwdParams p = bwd_params(q, k, v, dout, lse, delta, scale);
    p.dk = (float*)dk_acc.data;
    p.dv = (float*)dv_acc.data;
    p.dk_sB = dk_acc.sB; p.dk_sS = dk_acc.sS; p.dk_sH = dk_acc.sH;
    p.dv_sB = dv_acc.sB; p.dv_sS = dv_acc.sS; p.dv_sH = dv_acc.sH;
    p.km = km.data;
    p.km_sB = km.sB;
    // one workgroup per (128-key tile, KV head)
    p.n_tiles = (k.S + kBwdBlockN - 1) / kBwdBlockN;
    p.ds = (uint16_t*)ds;
    p.ds_nqt = ds_query_tiles(q.S);
    p.ds_nkg = ds_key_groups(k.S);
    if (dk_out && dv_out) {
        p.dk16 = (uint16_t*)dk_out->data;
        p.dv16 = (uint16_t*)dv_out->data;
        p.dk16_sB = dk_out->sB; p.dk16_sS = dk_out->sS; p.dk16_sH = dk_out->sH;
        p.dv16_sB = dv_out->sB; p.dv16_sS = dv_out->sS; p.dv16_sH = dv_out->sH;
    }
    const unsigned nb = (unsigned)p.n_tiles * k.H * q.B;
    if (q.D == 64) bwd_kv_bf16_kernel<64><<<nb, 64 * kBwdWaves * 2, 0, s>>>(p);
    else bwd_kv_bf16_kernel<128><<<nb, 64 * kBwdWaves * 2, 0, s>>>(p);
    return hipGetLastError();
}

hipError_t launch_bwd_dq_bf16(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const ra_tensor& dout,
                              const ra_lse& lse, const ra_lse& delta, const KeyMask& km, float scale,
                              const ra_tensor& dq_acc, hipStream_t s) {
    if (q.S == 0 || k.S == 0) return hipSuccess;
    BwdParams p = bwd_params(q, k, v, dout, lse, delta, scale);
    p.dq = (float*)dq_acc.data;
    p.dq_sB = dq_acc.sB; p.dq_sS = dq_acc.sS; p.dq_sH = dq_acc.sH;
    // one workgroup per (128-row query tile, query head)
    p.n_tiles = (q.S + kFwdBlockM - 1) / kFwdBlockM;
    const unsigned nb = (unsigned)p.n_tiles * q.H * q.B;
    p.km = km.data;
    p.km_sB = km.sB;
    if (km.data) {
        if (q.D == 64) bwd_dq_bf16_kernel<64, true><<<nb, 256, 0, s>>>(p);
        else bwd_dq_bf16_kernel<128, true><<<nb, 256, 0, s>>>(p);
    } else {
        if (q.D == 64) bwd_dq_bf16_kernel<64, false><<<nb, 256, 0, s>>>(p);
        else bwd_dq_bf16_kernel<128, false><<<nb, 256, 0, s>>>(p);
    }
    return hipGetLastError();
}

hipError_t launch_bwd_dqs_bf16(const ra_tensor& q, const ra_tensor& k, const void* ds, float scale,
                               const ra_tensor& dq_acc, hipStream_t s, bool dq_read, const ra_tensor* dq_out,
                               const KeyMask* km, const DqsChunk* more, int n_more) {
    if (q.S == 0 || k.S == 0) return hipSuccess;
    BwdParams p = bwd_params(q, k, k, q, ra_lse{}, ra_lse{}, scale);
    if (km) {
        p.km = km->data;
        p.km_sB = km->sB;
    }
    auto add = [&](const ra_tensor& kc, const void* dsc, const KeyMask* kmc) {
        const int j = p.n_dqs++;
        p.dqs_k[j] = (const uint16_t*)kc.data;
        p.dqs_kbytes[j] = span_bytes(kc.S, kc.sS, kc.D);
        p.dqs_Sk[j] = kc.S;
        p.dqs_nkg[j] = ds_key_groups(kc.S);
        p.dqs_ds[j] = (const uint16_t*)dsc;
        p.dqs_km[j] = kmc ? kmc->data : nullptr;
    };
    add(k, ds, km);
    for (int i = 0; i < n_more && p.n_dqs < kDqsMaxChunks; ++i)
        if (more[i].k.S > 0) add(more[i].k, more[i].ds, more[i].km);
    p.dq = (float*)dq_acc.data;
    p.dq_sB = dq_acc.sB; p.dq_sS = dq_acc.sS; p.dq_sH = dq_acc.sH;
    p.dq_read = dq_read ? 1 : 0;
    if (dq_out) {
        p.dq16 = (uint16_t*)dq_out->data;
        p.dq16_sB = dq_out->sB; p.dq16_sS = dq_out->sS; p.dq16_sH = dq_out->sH;
    }
    p.ds = (uint16_t*)ds;
    p.ds_nqt = ds_query_tiles(q.S);
    p.ds_nkg = ds_key_groups(k.S);
    // one workgroup per (kDqsWaves 64-row query tiles, query head)
    p.n_tiles = (p.ds_nqt + kDqsWaves - 1) / kDqsWaves;
    const unsigned nb = (unsigned)p.n_tiles * q.H * q.B;
    if (q.D == 64) bwd_dqs_bf16_kernel<64><<<nb, 64 * kDqsWaves, 0, s>>>(p);
    else bwd_dqs_bf16_kernel<128><<<nb, 64 * kDqsWaves, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace ra
