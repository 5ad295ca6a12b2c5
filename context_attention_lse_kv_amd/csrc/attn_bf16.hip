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
// its transposed operand is read with the gfx950 transposing LDS read.  The
// running max is only moved when a row's maximum grows by more than kRescale
// (base-2 units), so the output rescale is skipped on almost every tile.  The
// epilogue either writes the step's partial (normalised output, LSE) or merges it
// into the running fp32 (output, LSE) by LSE rescaling (the merge of the
// diffusers issue "Ring attention backward uses stale iteration-0 KV", table "How
// it surfaces per backend": ring needs LSE for partial-result merging).
//
// Backward (one launch per ring step, against that step's own K/V chunk - the
// point of that issue's "Root cause" and "Expected behavior"): a workgroup owns
// 128 keys of the chunk (32 per wavefront, K and V held in registers) for one
// query head and sweeps all query rows in LDS tiles of 64.  Per tile it
// recomputes S = Q K^T and dP = dO V^T with the final LSE and delta, forms P and
// dS, accumulates dV += P^T dO and dK += dS^T Q in registers, and adds
// dQ += dS K into the fp32 dQ accumulator with atomics after passing dS^T through
// LDS.  dK/dV are added atomically at the end because the query heads of a GQA
// group run in different workgroups.
//
// Both kernels stream their tiles with buffer loads (rows past the end of a
// slice read as zeros, so tails need no branches), keep the next tile in
// registers while the current one is computed, and double-buffer the LDS tiles
// so that one barrier per tile suffices.
#include "ra_device.h"

#define RA_LDS __attribute__((address_space(3)))

namespace ra {
namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef RA_LDS uint16_t lds_u16;

constexpr float kRescale = 8.0f;  // lazy-rescale threshold of the running max, in log2 units

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
    int B, Sq, Sk, Hq, G, n_ktiles;
    uint32_t q_bytes, do_bytes, k_bytes, v_bytes;
    float scale, c;
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

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane
// 4e+a passes the address of 4 consecutive bf16 (columns c0+4a..c0+4a+3) of row r0+e;
// lane i of the group then receives rows r0..r0+3 of column c0+i.
__device__ __forceinline__ u32x2_t lds_tr(const lds_u16* p) {
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((RA_LDS s16x4_t*)p);
    return __builtin_bit_cast(u32x2_t, v);
}

// MFMA operand of 8 bf16 made of rows r0..r0+3 and r0+8..r0+11 of column (c0 + lane)
// of a row-major LDS tile (pitch P): the k order of a 32x32 accumulator reused as an
// operand.  `p` already points at row r0 + e, column c0 + 4a of this lane.
template <int P>
__device__ __forceinline__ bf16x8_t lds_tr_split8(const lds_u16* p) {
    const u32x2_t lo = lds_tr(p), hi = lds_tr(p + 8 * P);
    return as_bf16x8(u32x4_t{lo[0], lo[1], hi[0], hi[1]});
}
// Same with 8 consecutive rows r0..r0+7.
template <int P>
__device__ __forceinline__ bf16x8_t lds_tr_cont8(const lds_u16* p) {
    const u32x2_t lo = lds_tr(p), hi = lds_tr(p + 4 * P);
    return as_bf16x8(u32x4_t{lo[0], lo[1], hi[0], hi[1]});
}

inline uint32_t span_bytes(int rows, int64_t stride, int D) {
    return rows <= 0 ? 0u : (uint32_t)(((int64_t)(rows - 1) * stride + D) * 2);
}

// ============================================================================ forward
template <int D, bool MERGE>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(FwdParams p) {
    constexpr int KS = D / 16, DB = D / 32, BN = kFwdBlockN, BM = kFwdBlockM;
    constexpr int KP = D + 8;    // K tile pitch (16-byte row reads)
    constexpr int VP = D + 16;   // V tile pitch (transposing reads)
    constexpr int KT = BN * KP, VT = BN * VP;
    constexpr int CH = BN * (D / 8) / 256;  // 16-byte chunks per thread per tile
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (KT + VT)];
    lds_u16* const Ks = (lds_u16*)smem;
    lds_u16* const Vs = Ks + 2 * KT;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int gq = lane >> 4, l16 = lane & 15;
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

    const uint16_t* kbase = p.k + (int64_t)b * p.k_sB + (int64_t)g * p.k_sH;
    const uint16_t* vbase = p.v + (int64_t)b * p.v_sB + (int64_t)g * p.v_sH;
    uint32_t vk[CH], vv[CH];
    int ko[CH], vo[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int c = tid + 256 * j, r = c / (D / 8), c8 = c % (D / 8);
        vk[j] = (uint32_t)((r * p.k_sS + 8 * c8) * 2);
        vv[j] = (uint32_t)((r * p.v_sS + 8 * c8) * 2);
        ko[j] = r * KP + 8 * c8;
        vo[j] = r * VP + 8 * c8;
    }
    u32x4_t kpre[CH], vpre[CH];
    // lane-constant parts of the transposing-read addresses of V
    const int vtr = (4 * hh + (l16 >> 2)) * VP + 16 * (gq & 1) + 4 * (l16 & 3);

    {
        const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kbase, 0, p.k_sS * 2, p.k_bytes);
        const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vbase, 0, p.v_sS * 2, p.v_bytes);
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            kpre[j] = bload16(rk, vk[j], 0);
            vpre[j] = bload16(rv, vv[j], 0);
        }
    }
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        *(RA_LDS u32x4_t*)(Ks + ko[j]) = kpre[j];
        *(RA_LDS u32x4_t*)(Vs + vo[j]) = vpre[j];
    }
    __syncthreads();

    const int ntiles = (p.Sk + BN - 1) / BN;
    for (int it = 0; it < ntiles; ++it) {
        const int buf = it & 1, n0 = it * BN;
        const bool more = it + 1 < ntiles;
        if (more) {
            const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kbase, n0 + BN, p.k_sS * 2, p.k_bytes);
            const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vbase, n0 + BN, p.v_sS * 2, p.v_bytes);
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                kpre[j] = bload16(rk, vk[j], 0);
                vpre[j] = bload16(rv, vv[j], 0);
            }
        }
        const lds_u16* kb = Ks + buf * KT;
        const lds_u16* vb = Vs + buf * VT;

        // S^T (keys x rows) for this wave's 32 rows: two 32-key blocks
        f32x16_t sacc[2];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
            sacc[kb2] = f32x16_t{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                sacc[kb2] = mfma32(lds_b128(kb + (kb2 * 32 + l32) * KP + 16 * ks + 8 * hh), qreg[ks], sacc[kb2]);
        }
        if (n0 + BN > p.Sk) {  // last tile: keys past the chunk read as zero; mask them
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (n0 + kb2 * 32 + 8 * (r / 4) + 4 * hh + (r % 4) >= p.Sk) sacc[kb2][r] = -INFINITY;
        }
        // online softmax in base 2 on t = s * scale * log2(e), with a lazily moved max
        float mx = -INFINITY;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb2][r]);
        mx = fmaxf(mx, swap_half(mx)) * p.c;
        if (__builtin_amdgcn_ballot_w64(mx > m + kRescale) != 0) {
            const float m_new = fmaxf(m, mx);
            const float alpha = __builtin_amdgcn_exp2f(m - m_new);
            l *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            m = m_new;
        }
        u32x4_t pk[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 8 * (t % 2) + 2 * j;
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t / 2][r], p.c, -m));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t / 2][r + 1], p.c, -m));
                l += p0 + p1;
                pk[t][j] = pack_bf16x2(p0, p1);
            }
        // O^T += V^T P^T over the tile's 64 keys (4 k-steps of 16)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const bf16x8_t pb = as_bf16x8(pk[t]);
#pragma unroll
            for (int db = 0; db < DB; ++db)
                oacc[db] = mfma32(lds_tr_split8<VP>(vb + vtr + 16 * t * VP + 32 * db), pb, oacc[db]);
        }
        if (more) {
            lds_u16* kn = Ks + (buf ^ 1) * KT;
            lds_u16* vn = Vs + (buf ^ 1) * VT;
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                *(RA_LDS u32x4_t*)(kn + ko[j]) = kpre[j];
                *(RA_LDS u32x4_t*)(vn + vo[j]) = vpre[j];
            }
        }
        __syncthreads();
    }

    l += swap_half(l);
    if (!row_ok) return;
    const float inv_l = 1.f / l;
    const float lse_c = m * kLn2 + logf(l);
    float* orow = p.out + (int64_t)b * p.o_sB + (int64_t)row * p.o_sS + (int64_t)h * p.o_sH;
    float* lp = p.lse + (int64_t)b * p.l_sB + (int64_t)h * p.l_sH + row;
    if (!MERGE) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4_t v4 = {oacc[db][4 * g4] * inv_l, oacc[db][4 * g4 + 1] * inv_l,
                                    oacc[db][4 * g4 + 2] * inv_l, oacc[db][4 * g4 + 3] * inv_l};
                *(f32x4_t*)(orow + 32 * db + 8 * g4 + 4 * hh) = v4;
            }
        if (hh == 0) *lp = lse_c;
    } else {
        // both lanes of the row (l and l^32) read lse_acc before lane l writes it (same wavefront)
        const float la = *lp;
        const float mm = fmaxf(la, lse_c);
        const float ea = expf(la - mm), ec = expf(lse_c - mm);
        const float sum = ea + ec;
        const float wa = ea / sum, wc = ec / sum * inv_l;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                f32x4_t* po = (f32x4_t*)(orow + 32 * db + 8 * g4 + 4 * hh);
                const f32x4_t old = *po;
                f32x4_t v4;
#pragma unroll
                for (int j = 0; j < 4; ++j) v4[j] = (wa == 0.f ? 0.f : wa * old[j]) + wc * oacc[db][4 * g4 + j];
                *po = v4;
            }
        if (hh == 0) *lp = mm + logf(sum);
    }
}

// ============================================================================ backward
template <int D>
__global__ __launch_bounds__(256, 1) void bwd_bf16_kernel(BwdParams p) {
    constexpr int KS = D / 16, DB = D / 32, BN = kBwdBlockN, BM = kBwdBlockM;
    constexpr int RB = BM / 32;       // 32-row blocks per Q tile
    constexpr int QP = D + 8;         // Q / dO tile pitch (row reads and transposing reads)
    constexpr int KTP = D + 16;       // K tile pitch (transposing reads)
    constexpr int SP = BM + 16;       // dS^T tile pitch ([key][row], transposing reads)
    constexpr int QT = BM * QP;
    constexpr int CHQ = BM * (D / 8) / 256;
    constexpr int CHK = BN * (D / 8) / 256;
    constexpr int DQ_TILES = RB * DB / 4;  // dQ 32x32 tiles per wavefront
    __shared__ __attribute__((aligned(16))) uint16_t smem[BN * KTP + 4 * QT + BN * SP];
    __shared__ __attribute__((aligned(16))) float stat[2][2][BM];  // [buffer][lse*log2e | delta][row]
    lds_u16* const Ks = (lds_u16*)smem;
    lds_u16* const Qs = Ks + BN * KTP;   // [2][BM][QP]
    lds_u16* const Os = Qs + 2 * QT;     // [2][BM][QP]
    lds_u16* const dSt = Os + 2 * QT;    // [BN][SP]

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int gq = lane >> 4, l16 = lane & 15;
    const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x);
    const int kt = (int)(logical % p.n_ktiles);
    const int rest = (int)(logical / p.n_ktiles);
    const int h = rest % p.Hq, b = rest / p.Hq, g = h / p.G;
    const int n0 = kt * BN;
    const int key = n0 + 32 * w + l32;  // this lane's key (column of S/dP, row of dK/dV)
    const bool key_ok = key < p.Sk;
    const bool keys_partial = n0 + BN > p.Sk;

    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + (int64_t)b * p.k_sB + (int64_t)g * p.k_sH, p.k_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + (int64_t)b * p.v_sB + (int64_t)g * p.v_sH, p.v_bytes);
    const uint16_t* qbase = p.q + (int64_t)b * p.q_sB + (int64_t)h * p.q_sH;
    const uint16_t* obase = p.dout + (int64_t)b * p.do_sB + (int64_t)h * p.do_sH;
    const float* lbase = p.lse + (int64_t)b * p.l_sB + (int64_t)h * p.l_sH;
    const float* dbase = p.delta + (int64_t)b * p.d_sB + (int64_t)h * p.d_sH;

    // K rows of the workgroup (for dQ), and this lane's K and V rows as MFMA operands
#pragma unroll
    for (int j = 0; j < CHK; ++j) {
        const int c = tid + 256 * j, r = c / (D / 8), c8 = c % (D / 8);
        *(RA_LDS u32x4_t*)(Ks + r * KTP + 8 * c8) = bload16(rk, (uint32_t)(((n0 + r) * p.k_sS + 8 * c8) * 2), 0);
    }
    bf16x8_t kreg[KS], vreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        kreg[ks] = as_bf16x8(bload16(rk, (uint32_t)((key * p.k_sS + 16 * ks + 8 * hh) * 2), 0));
        vreg[ks] = as_bf16x8(bload16(rv, (uint32_t)((key * p.v_sS + 16 * ks + 8 * hh) * 2), 0));
    }
    f32x16_t dkacc[DB], dvacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        dkacc[db] = f32x16_t{};
        dvacc[db] = f32x16_t{};
    }

    uint32_t vq[CHQ], vo[CHQ];
    int lo[CHQ];
#pragma unroll
    for (int j = 0; j < CHQ; ++j) {
        const int c = tid + 256 * j, r = c / (D / 8), c8 = c % (D / 8);
        vq[j] = (uint32_t)((r * p.q_sS + 8 * c8) * 2);
        vo[j] = (uint32_t)((r * p.do_sS + 8 * c8) * 2);
        lo[j] = r * QP + 8 * c8;
    }
    u32x4_t qpre[CHQ], opre[CHQ];
    float lpre = 0.f, dpre = 0.f;
    auto issue = [&](int it) {
        const int r0 = it * BM;
        const __amdgpu_buffer_rsrc_t rq = tile_rsrc(qbase, r0, p.q_sS * 2, p.q_bytes);
        const __amdgpu_buffer_rsrc_t ro = tile_rsrc(obase, r0, p.do_sS * 2, p.do_bytes);
#pragma unroll
        for (int j = 0; j < CHQ; ++j) {
            qpre[j] = bload16(rq, vq[j], 0);
            opre[j] = bload16(ro, vo[j], 0);
        }
        if (tid < BM) {
            const uint32_t nbytes = (uint32_t)p.Sq * 4;
            lpre = bload4f(tile_rsrc(lbase, r0, 4, nbytes), (uint32_t)tid * 4, 0);
            dpre = bload4f(tile_rsrc(dbase, r0, 4, nbytes), (uint32_t)tid * 4, 0);
        }
    };
    auto commit = [&](int buf) {
#pragma unroll
        for (int j = 0; j < CHQ; ++j) {
            *(RA_LDS u32x4_t*)(Qs + buf * QT + lo[j]) = qpre[j];
            *(RA_LDS u32x4_t*)(Os + buf * QT + lo[j]) = opre[j];
        }
        if (tid < BM) {
            stat[buf][0][tid] = lpre * kLog2e;
            stat[buf][1][tid] = dpre;
        }
    };
    // lane-constant parts of transposing-read addresses
    const int trQ = (4 * hh + (l16 >> 2)) * QP + 16 * (gq & 1) + 4 * (l16 & 3);       // dO^T / Q^T operands
    const int trS = (8 * hh + (l16 >> 2)) * SP + 16 * (gq & 1) + 4 * (l16 & 3);       // dS operand
    const int trK = (8 * hh + (l16 >> 2)) * KTP + 16 * (gq & 1) + 4 * (l16 & 3);      // K operand of dQ
    float* dqbase = p.dq + (int64_t)b * p.dq_sB + (int64_t)h * p.dq_sH;

    issue(0);
    commit(0);
    __syncthreads();
    const int ntiles = (p.Sq + BM - 1) / BM;
    for (int it = 0; it < ntiles; ++it) {
        const int buf = it & 1, i0 = it * BM;
        const bool more = it + 1 < ntiles;
        if (more) issue(it + 1);
        const lds_u16* qb = Qs + buf * QT;
        const lds_u16* ob = Os + buf * QT;

        u32x4_t pp[RB][2], pd[RB][2];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            f32x16_t sacc = f32x16_t{}, dpacc = f32x16_t{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                sacc = mfma32(lds_b128(qb + (32 * rb + l32) * QP + 16 * ks + 8 * hh), kreg[ks], sacc);
                dpacc = mfma32(lds_b128(ob + (32 * rb + l32) * QP + 16 * ks + 8 * hh), vreg[ks], dpacc);
            }
            // lane = key, register r = row 32*rb + 8*(r/4) + 4*hh + r%4
            float pv[16], dsv[16];
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4_t l2 = *(const RA_LDS f32x4_t*)&stat[buf][0][32 * rb + 8 * g4 + 4 * hh];
                const f32x4_t dl = *(const RA_LDS f32x4_t*)&stat[buf][1][32 * rb + 8 * g4 + 4 * hh];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 4 * g4 + j;
                    pv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], p.c, -l2[j]));
                }
                if (keys_partial) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) pv[4 * g4 + j] = key_ok ? pv[4 * g4 + j] : 0.f;
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 4 * g4 + j;
                    dsv[r] = pv[r] * (dpacc[r] - dl[j]);
                }
            }
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pp[rb][t2][j] = pack_bf16x2(pv[8 * t2 + 2 * j], pv[8 * t2 + 2 * j + 1]);
                    pd[rb][t2][j] = pack_bf16x2(dsv[8 * t2 + 2 * j], dsv[8 * t2 + 2 * j + 1]);
                }
            // dS^T rows for the dQ product: 4 consecutive query rows per 8-byte write
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
                *(RA_LDS u32x2_t*)(dSt + (32 * w + l32) * SP + 32 * rb + 8 * g4 + 4 * hh) =
                    u32x2_t{pd[rb][g4 / 2][2 * (g4 % 2)], pd[rb][g4 / 2][2 * (g4 % 2) + 1]};
        }
        // dV += P^T dO, dK += dS^T Q (k = query rows, 2 k-steps of 16 per row block)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
                const bf16x8_t pa = as_bf16x8(pp[rb][t2]);
                const bf16x8_t da = as_bf16x8(pd[rb][t2]);
                const int off = trQ + (32 * rb + 16 * t2) * QP;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    dvacc[db] = mfma32(pa, lds_tr_split8<QP>(ob + off + 32 * db), dvacc[db]);
                    dkacc[db] = mfma32(da, lds_tr_split8<QP>(qb + off + 32 * db), dkacc[db]);
                }
            }
        __syncthreads();
        // dQ[rows][d] += scale * dS K over the workgroup's 128 keys
        const bool rows_full = i0 + BM <= p.Sq;
#pragma unroll
        for (int j = 0; j < DQ_TILES; ++j) {
            const int ti = w + 4 * j;
            const int rb = ti % RB, db = ti / RB;
            f32x16_t acc = f32x16_t{};
#pragma unroll
            for (int t = 0; t < BN / 16; ++t)
                acc = mfma32(lds_tr_cont8<SP>(dSt + trS + 16 * t * SP + 32 * rb),
                             lds_tr_cont8<KTP>(Ks + trK + 16 * t * KTP + 32 * db), acc);
            float* dst = dqbase + (int64_t)(i0 + 32 * rb + 4 * hh) * p.dq_sS + 32 * db + l32;
            if (rows_full) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    unsafeAtomicAdd(dst + (int64_t)(8 * (r / 4) + (r % 4)) * p.dq_sS, p.scale * acc[r]);
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (i0 + 32 * rb + 8 * (r / 4) + 4 * hh + (r % 4) < p.Sq)
                        unsafeAtomicAdd(dst + (int64_t)(8 * (r / 4) + (r % 4)) * p.dq_sS, p.scale * acc[r]);
            }
        }
        if (more) commit(buf ^ 1);
        __syncthreads();
    }

    // dK, dV rows of this wave's 32 keys: lane = d column, register r = key 8*(r/4) + 4*hh + r%4
    float* dkb = p.dk + (int64_t)b * p.dk_sB + (int64_t)g * p.dk_sH + (int64_t)(n0 + 32 * w + 4 * hh) * p.dk_sS + l32;
    float* dvb = p.dv + (int64_t)b * p.dv_sB + (int64_t)g * p.dv_sH + (int64_t)(n0 + 32 * w + 4 * hh) * p.dv_sS + l32;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kr = 8 * (r / 4) + (r % 4);
            if (!keys_partial || n0 + 32 * w + 4 * hh + kr < p.Sk) {
                unsafeAtomicAdd(dkb + (int64_t)kr * p.dk_sS + 32 * db, p.scale * dkacc[db][r]);
                unsafeAtomicAdd(dvb + (int64_t)kr * p.dv_sS + 32 * db, dvacc[db][r]);
            }
        }
}

}  // namespace

hipError_t launch_fwd_chunk_bf16(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, float scale,
                                 const ra_tensor& out, const ra_lse& lse, int merge, hipStream_t s) {
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
    if (q.D == 64) {
        if (merge) fwd_bf16_kernel<64, true><<<nb, 256, 0, s>>>(p);
        else fwd_bf16_kernel<64, false><<<nb, 256, 0, s>>>(p);
    } else {
        if (merge) fwd_bf16_kernel<128, true><<<nb, 256, 0, s>>>(p);
        else fwd_bf16_kernel<128, false><<<nb, 256, 0, s>>>(p);
    }
    return hipGetLastError();
}

hipError_t launch_bwd_chunk_bf16(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const ra_tensor& dout,
                                 const ra_lse& lse, const ra_lse& delta, float scale, const ra_tensor& dq_acc,
                                 const ra_tensor& dk_acc, const ra_tensor& dv_acc, hipStream_t s) {
    if (q.S == 0 || k.S == 0) return hipSuccess;
    BwdParams p;
    p.q = (const uint16_t*)q.data;
    p.k = (const uint16_t*)k.data;
    p.v = (const uint16_t*)v.data;
    p.dout = (const uint16_t*)dout.data;
    p.lse = lse.data;
    p.delta = delta.data;
    p.dq = (float*)dq_acc.data;
    p.dk = (float*)dk_acc.data;
    p.dv = (float*)dv_acc.data;
    p.q_sB = q.sB; p.q_sS = q.sS; p.q_sH = q.sH;
    p.k_sB = k.sB; p.k_sS = k.sS; p.k_sH = k.sH;
    p.v_sB = v.sB; p.v_sS = v.sS; p.v_sH = v.sH;
    p.do_sB = dout.sB; p.do_sS = dout.sS; p.do_sH = dout.sH;
    p.l_sB = lse.sB; p.l_sH = lse.sH;
    p.d_sB = delta.sB; p.d_sH = delta.sH;
    p.dq_sB = dq_acc.sB; p.dq_sS = dq_acc.sS; p.dq_sH = dq_acc.sH;
    p.dk_sB = dk_acc.sB; p.dk_sS = dk_acc.sS; p.dk_sH = dk_acc.sH;
    p.dv_sB = dv_acc.sB; p.dv_sS = dv_acc.sS; p.dv_sH = dv_acc.sH;
    p.B = q.B; p.Sq = q.S; p.Sk = k.S; p.Hq = q.H; p.G = q.H / k.H;
    p.n_ktiles = (k.S + kBwdBlockN - 1) / kBwdBlockN;
    p.q_bytes = span_bytes(q.S, q.sS, q.D);
    p.do_bytes = span_bytes(dout.S, dout.sS, dout.D);
    p.k_bytes = span_bytes(k.S, k.sS, k.D);
    p.v_bytes = span_bytes(v.S, v.sS, v.D);
    p.scale = scale;
    p.c = scale * 1.4426950408889634f;
    const unsigned nb = (unsigned)p.n_ktiles * q.H * q.B;
    if (q.D == 64) bwd_bf16_kernel<64><<<nb, 256, 0, s>>>(p);
    else bwd_bf16_kernel<128><<<nb, 256, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace ra
