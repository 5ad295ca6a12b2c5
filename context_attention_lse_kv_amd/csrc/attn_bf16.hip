// bf16 chunk steps of ring attention on gfx950 matrix cores (MFMA 32x32x16 bf16,
// fp32 accumulate).
//
// Forward (one launch per ring step): a workgroup of 4 wavefronts owns 128 query
// rows of one (batch, query head); each wavefront keeps its 32 rows of Q in
// registers and sweeps the chunk's keys in LDS tiles of 64.  Scores are formed
// transposed, S^T = K Q^T, so that a lane owns one query row: the online-softmax
// state (running max m, running sum l) and the rescale of the output are
// lane-local, and the probabilities P^T come out of the MFMA already in the
// operand layout of the second product O^T += V^T P^T.  V is written to LDS
// transposed ([d][key]) while it is staged.  The epilogue either writes the
// step's partial (normalised output, LSE) or merges it into the running fp32
// (output, LSE) by LSE rescaling (the merge of the diffusers issue "Ring
// attention backward uses stale iteration-0 KV", table "How it surfaces per
// backend": ring needs LSE for partial-result merging).
//
// Backward (one launch per ring step, against that step's own K/V chunk - the
// point of that issue's "Root cause" and "Expected behavior"): a workgroup owns
// 128 keys of the chunk (32 per wavefront, K and V held in registers) for one
// query head and sweeps all query rows in LDS tiles of 64.  Per tile it
// recomputes S = Q K^T and dP = dO V^T with the final LSE and delta, forms P and
// dS, accumulates dV += P^T dO and dK += dS^T Q in registers, and adds
// dQ += dS K into the fp32 dQ accumulator with atomics after passing dS through
// LDS.  dK/dV are added atomically at the end because the query heads of a GQA
// group run in different workgroups.
#include "ra_device.h"

namespace ra {
namespace {

struct FwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    float* out;
    float* lse;
    int64_t q_sB, q_sS, q_sH, k_sB, k_sS, k_sH, v_sB, v_sS, v_sH, o_sB, o_sS, o_sH, l_sB, l_sH;
    int B, Sq, Sk, Hq, G, n_qtiles;
    float c;  // scale * log2(e)
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
    float scale, c;
};

__device__ __forceinline__ u32x4_t ldg16(const uint16_t* p) { return *(const u32x4_t*)p; }

// Pack the d-th column of 4 rows (each row: 8 bf16 in a u32x4) into 4 consecutive
// bf16 (8 bytes): for d = 2p + 0 take the low halves, for 2p + 1 the high halves.
__device__ __forceinline__ u32x2_t col4(const u32x4_t (&w)[4], int p, bool hi) {
    const uint32_t sel = hi ? 0x07060302u : 0x05040100u;
    u32x2_t r;
    r[0] = __builtin_amdgcn_perm(w[1][p], w[0][p], sel);
    r[1] = __builtin_amdgcn_perm(w[3][p], w[2][p], sel);
    return r;
}

// Stage rows [r0, r0 + 4*n4) x D of a [rows][D] bf16 slice: 4 rows x 8 columns per
// work item.  Writes a row-major copy (pitch RP) if RM, and a transposed copy
// ([d][row], pitch TP) if TR.  Rows >= nrows are zero.
template <int D, int RP, int TP, bool RM, bool TR>
__device__ __forceinline__ void stage_tile(uint16_t* rm, uint16_t* tr, const uint16_t* base, int64_t sS, int r0,
                                           int nrows, int n4) {
    for (int it = threadIdx.x; it < n4 * (D / 8); it += 256) {
        const int rg = it / (D / 8), c8 = it % (D / 8);
        u32x4_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = r0 + 4 * rg + j;
            if (r < nrows) {
                w[j] = ldg16(base + (int64_t)r * sS + 8 * c8);
            } else {
                w[j] = u32x4_t{0u, 0u, 0u, 0u};
            }
        }
        if (RM) {
#pragma unroll
            for (int j = 0; j < 4; ++j) *(u32x4_t*)&rm[(4 * rg + j) * RP + 8 * c8] = w[j];
        }
        if (TR) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                *(u32x2_t*)&tr[(8 * c8 + 2 * p) * TP + 4 * rg] = col4(w, p, false);
                *(u32x2_t*)&tr[(8 * c8 + 2 * p + 1) * TP + 4 * rg] = col4(w, p, true);
            }
        }
    }
}

// Operand of 8 bf16 made of two 4-element runs at p and p + 8 (the k order that a
// 32x32 accumulator's registers follow when reused as an operand).
__device__ __forceinline__ bf16x8_t ld_split8(const uint16_t* p) {
    const u32x2_t lo = *(const u32x2_t*)p;
    const u32x2_t hi = *(const u32x2_t*)(p + 8);
    return as_bf16x8(u32x4_t{lo[0], lo[1], hi[0], hi[1]});
}

// ============================================================================ forward
template <int D, bool MERGE>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(FwdParams p) {
    constexpr int KS = D / 16, DB = D / 32, BN = kFwdBlockN, BM = kFwdBlockM;
    constexpr int KP = D + 8;   // K tile pitch
    constexpr int VP = BN + 8;  // V^T tile pitch
    __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * KP];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VP];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
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
            qreg[ks] = row_ok ? as_bf16x8(ldg16(qrow + 16 * ks + 8 * hh)) : as_bf16x8(u32x4_t{0u, 0u, 0u, 0u});
    }
    f32x16_t oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16_t{};
    float m = -INFINITY, l = 0.f;

    const uint16_t* kbase = p.k + (int64_t)b * p.k_sB + (int64_t)g * p.k_sH;
    const uint16_t* vbase = p.v + (int64_t)b * p.v_sB + (int64_t)g * p.v_sH;

    for (int n0 = 0; n0 < p.Sk; n0 += BN) {
        __syncthreads();
        stage_tile<D, KP, VP, true, false>(Ks, nullptr, kbase, p.k_sS, n0, p.Sk, BN / 4);
        stage_tile<D, KP, VP, false, true>(nullptr, Vt, vbase, p.v_sS, n0, p.Sk, BN / 4);
        __syncthreads();

        // S^T (keys x rows) for this wave's 32 rows: two 32-key blocks
        f32x16_t sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            sacc[kb] = f32x16_t{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8_t a = *(const bf16x8_t*)&Ks[(kb * 32 + l32) * KP + 16 * ks + 8 * hh];
                sacc[kb] = mfma32(a, qreg[ks], sacc[kb]);
            }
        }
        if (n0 + BN > p.Sk) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = n0 + kb * 32 + 8 * (r / 4) + 4 * hh + (r % 4);
                    if (key >= p.Sk) sacc[kb][r] = -INFINITY;
                }
        }
        // online softmax in base 2 on scaled scores t = s * scale * log2(e)
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
        mx = fmaxf(mx, swap_half(mx));
        const float m_new = fmaxf(m, mx * p.c);
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        uint32_t pk[2][8];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], p.c, -m_new));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r + 1], p.c, -m_new));
                l += p0 + p1;
                pk[kb][r / 2] = pack_bf16x2(p0, p1);
            }
        m = m_new;
        // O^T += V^T P^T over the tile's 64 keys (4 k-steps of 16)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int kb = t / 2, base = 4 * (t % 2);
            const bf16x8_t pb = as_bf16x8(u32x4_t{pk[kb][base], pk[kb][base + 1], pk[kb][base + 2], pk[kb][base + 3]});
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16x8_t va = ld_split8(&Vt[(32 * db + l32) * VP + 16 * t + 4 * hh]);
                oacc[db] = mfma32(va, pb, oacc[db]);
            }
        }
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
    constexpr int RB = BM / 32;     // 32-row blocks per Q tile
    constexpr int QP = D + 8;       // row-major Q / dO pitch
    constexpr int TP = BM + 8;      // transposed Q / dO pitch
    constexpr int SP = BN + 8;      // dS pitch
    constexpr int KTP = BN + 8;     // K^T pitch
    constexpr int DQ_TILES = RB * DB / 4;  // dQ 32x32 tiles per wavefront
    __shared__ __attribute__((aligned(16))) uint16_t Qs[BM * QP];
    __shared__ __attribute__((aligned(16))) uint16_t Os[BM * QP];
    __shared__ __attribute__((aligned(16))) uint16_t Qt[D * TP];
    __shared__ __attribute__((aligned(16))) uint16_t Ot[D * TP];
    __shared__ __attribute__((aligned(16))) uint16_t dSs[BM * SP];
    __shared__ __attribute__((aligned(16))) uint16_t Kt[D * KTP];
    __shared__ float lse2s[BM];
    __shared__ float dls[BM];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x);
    const int kt = (int)(logical % p.n_ktiles);
    const int rest = (int)(logical / p.n_ktiles);
    const int h = rest % p.Hq, b = rest / p.Hq, g = h / p.G;
    const int n0 = kt * BN;
    const int key = n0 + 32 * w + l32;  // this lane's key (for S/dP columns and dK/dV rows)
    const bool key_ok = key < p.Sk;

    const uint16_t* kbase = p.k + (int64_t)b * p.k_sB + (int64_t)g * p.k_sH;
    const uint16_t* vbase = p.v + (int64_t)b * p.v_sB + (int64_t)g * p.v_sH;
    const uint16_t* qbase = p.q + (int64_t)b * p.q_sB + (int64_t)h * p.q_sH;
    const uint16_t* obase = p.dout + (int64_t)b * p.do_sB + (int64_t)h * p.do_sH;

    // K^T of the workgroup's keys for the dQ product; K and V rows of this lane's key
    stage_tile<D, QP, KTP, false, true>(nullptr, Kt, kbase, p.k_sS, n0, p.Sk, BN / 4);
    bf16x8_t kreg[KS], vreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const u32x4_t z = {0u, 0u, 0u, 0u};
        kreg[ks] = as_bf16x8(key_ok ? ldg16(kbase + (int64_t)key * p.k_sS + 16 * ks + 8 * hh) : z);
        vreg[ks] = as_bf16x8(key_ok ? ldg16(vbase + (int64_t)key * p.v_sS + 16 * ks + 8 * hh) : z);
    }
    f32x16_t dkacc[DB], dvacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        dkacc[db] = f32x16_t{};
        dvacc[db] = f32x16_t{};
    }
    const float* lrow = p.lse + (int64_t)b * p.l_sB + (int64_t)h * p.l_sH;
    const float* drow = p.delta + (int64_t)b * p.d_sB + (int64_t)h * p.d_sH;
    float* dqbase = p.dq + (int64_t)b * p.dq_sB + (int64_t)h * p.dq_sH;

    for (int i0 = 0; i0 < p.Sq; i0 += BM) {
        __syncthreads();
        stage_tile<D, QP, TP, true, true>(Qs, Qt, qbase, p.q_sS, i0, p.Sq, BM / 4);
        stage_tile<D, QP, TP, true, true>(Os, Ot, obase, p.do_sS, i0, p.Sq, BM / 4);
        if (tid < BM) {
            const int r = i0 + tid;
            lse2s[tid] = r < p.Sq ? lrow[r] * kLog2e : INFINITY;
            dls[tid] = r < p.Sq ? drow[r] : 0.f;
        }
        __syncthreads();

#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            f32x16_t sacc = f32x16_t{}, dpacc = f32x16_t{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8_t qa = *(const bf16x8_t*)&Qs[(32 * rb + l32) * QP + 16 * ks + 8 * hh];
                sacc = mfma32(qa, kreg[ks], sacc);
                const bf16x8_t oa = *(const bf16x8_t*)&Os[(32 * rb + l32) * QP + 16 * ks + 8 * hh];
                dpacc = mfma32(oa, vreg[ks], dpacc);
            }
            // lane = key, register r = row 32*rb + 8*(r/4) + 4*hh + r%4
            uint32_t pp[8], pd[8];
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                float pv[2], dsv[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int rr = 32 * rb + 8 * ((r + j) / 4) + 4 * hh + ((r + j) % 4);
                    float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r + j], p.c, -lse2s[rr]));
                    pr = key_ok ? pr : 0.f;
                    pv[j] = pr;
                    dsv[j] = pr * (dpacc[r + j] - dls[rr]);
                    dSs[rr * SP + 32 * w + l32] = (uint16_t)(pack_bf16x2(dsv[j], 0.f) & 0xffffu);
                }
                pp[r / 2] = pack_bf16x2(pv[0], pv[1]);
                pd[r / 2] = pack_bf16x2(dsv[0], dsv[1]);
            }
            // dV += P^T dO, dK += dS^T Q over this row block (2 k-steps of 16 rows)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
                const bf16x8_t pa = as_bf16x8(u32x4_t{pp[4 * t2], pp[4 * t2 + 1], pp[4 * t2 + 2], pp[4 * t2 + 3]});
                const bf16x8_t da = as_bf16x8(u32x4_t{pd[4 * t2], pd[4 * t2 + 1], pd[4 * t2 + 2], pd[4 * t2 + 3]});
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int off = (32 * db + l32) * TP + 32 * rb + 16 * t2 + 4 * hh;
                    dvacc[db] = mfma32(pa, ld_split8(&Ot[off]), dvacc[db]);
                    dkacc[db] = mfma32(da, ld_split8(&Qt[off]), dkacc[db]);
                }
            }
        }
        __syncthreads();
        // dQ[rows][d] += scale * dS K over the workgroup's 128 keys
#pragma unroll
        for (int j = 0; j < DQ_TILES; ++j) {
            const int ti = w + 4 * j;
            const int rb = ti % RB, db = ti / RB;
            f32x16_t acc = f32x16_t{};
#pragma unroll
            for (int t = 0; t < BN / 16; ++t) {
                const bf16x8_t a = *(const bf16x8_t*)&dSs[(32 * rb + l32) * SP + 16 * t + 8 * hh];
                const bf16x8_t bk = *(const bf16x8_t*)&Kt[(32 * db + l32) * KTP + 16 * t + 8 * hh];
                acc = mfma32(a, bk, acc);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rr = i0 + 32 * rb + 8 * (r / 4) + 4 * hh + (r % 4);
                if (rr < p.Sq) unsafeAtomicAdd(dqbase + (int64_t)rr * p.dq_sS + 32 * db + l32, p.scale * acc[r]);
            }
        }
    }

    // dK, dV rows of this wave's 32 keys: lane = d column, register r = key 8*(r/4) + 4*hh + r%4
    float* dkb = p.dk + (int64_t)b * p.dk_sB + (int64_t)g * p.dk_sH;
    float* dvb = p.dv + (int64_t)b * p.dv_sB + (int64_t)g * p.dv_sH;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kk = n0 + 32 * w + 8 * (r / 4) + 4 * hh + (r % 4);
            if (kk < p.Sk) {
                unsafeAtomicAdd(dkb + (int64_t)kk * p.dk_sS + 32 * db + l32, p.scale * dkacc[db][r]);
                unsafeAtomicAdd(dvb + (int64_t)kk * p.dv_sS + 32 * db + l32, dvacc[db][r]);
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
    p.scale = scale;
    p.c = scale * 1.4426950408889634f;
    const unsigned nb = (unsigned)p.n_ktiles * q.H * q.B;
    if (q.D == 64) bwd_bf16_kernel<64><<<nb, 256, 0, s>>>(p);
    else bwd_bf16_kernel<128><<<nb, 256, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace ra
