// fp32 chunk steps (no bf16 anywhere, accurate expf/logf): the fp32 instantiation
// of the ring path, for inputs that are fp32 end to end.  These are VALU kernels:
// a query row (forward, dQ) or a key row (dK/dV) is owned by T = D/32 lanes, each
// holding 32 of its D elements; dot products are reduced across those lanes.
// K/V (or Q/dO) tiles are staged in LDS and read by broadcast.  With a key mask,
// masked keys are skipped (forward, dQ) or get no dK/dV (dK/dV kernel); a forward row
// that meets no valid key in the chunk yields the merge identity (out 0, lse -inf).
#include "ra_device.h"

namespace ra {
namespace {

constexpr int kThreads = 128;
constexpr int kTile = 32;  // rows per LDS tile
constexpr int kSub = 32;   // elements of a row held by one lane

__device__ __forceinline__ bool key_on(const KeyMask& km, int b, int key) {
    return km.data == nullptr || km.data[(int64_t)b * km.sB + key] != 0;
}

__device__ __forceinline__ const float* rowp(const ra_tensor& t, int b, int s, int h) {
    return (const float*)t.data + (int64_t)b * t.sB + (int64_t)s * t.sS + (int64_t)h * t.sH;
}

template <int T>
__device__ __forceinline__ float group_sum(float x) {
    for (int w = T / 2; w >= 1; w /= 2) x += __shfl_xor(x, w, 64);
    return x;
}

// Loads rows [r0, r0+kTile) (clipped to n) of the (b, h) slice of t into lds[kTile][D].
template <int D>
__device__ __forceinline__ void stage_rows(float (*lds)[D], const ra_tensor& t, int b, int h, int r0, int n) {
    for (int i = threadIdx.x; i < kTile * (D / 4); i += kThreads) {
        const int r = i / (D / 4), c = i % (D / 4);
        f32x4_t v = {0.f, 0.f, 0.f, 0.f};
        if (r0 + r < n) v = ((const f32x4_t*)rowp(t, b, r0 + r, h))[c];
        *(f32x4_t*)&lds[r][4 * c] = v;
    }
}

// ---------------------------------------------------------------- forward chunk step
template <int D>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(ra_tensor q, ra_tensor k, ra_tensor v, KeyMask km,
                                                           float scale, ra_tensor out, ra_lse lse, int merge) {
    constexpr int T = D / kSub;
    constexpr int RowsPerBlock = kThreads / T;
    __shared__ float Ks[kTile][D];
    __shared__ float Vs[kTile][D];
    const int b = blockIdx.z, h = blockIdx.y;
    const int g = h / (q.H / k.H);
    const int part = threadIdx.x % T;
    const int row = blockIdx.x * RowsPerBlock + threadIdx.x / T;
    const bool valid = row < q.S;
    float qr[kSub], o[kSub];
    for (int j = 0; j < kSub; ++j) {
        qr[j] = valid ? rowp(q, b, row, h)[part * kSub + j] : 0.f;
        o[j] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for (int n0 = 0; n0 < k.S; n0 += kTile) {
        __syncthreads();
        stage_rows<D>(Ks, k, b, g, n0, k.S);
        stage_rows<D>(Vs, v, b, g, n0, k.S);
        __syncthreads();
        const int nk = min(kTile, k.S - n0);
        for (int j = 0; j < nk; ++j) {
            if (!key_on(km, b, n0 + j)) continue;
            float s = 0.f;
            for (int e = 0; e < kSub; ++e) s += qr[e] * Ks[j][part * kSub + e];
            s = group_sum<T>(s) * scale;
            if (s > m) {  // online softmax: rescale the running sum when the max grows
                const float alpha = expf(m - s);
                l *= alpha;
                for (int e = 0; e < kSub; ++e) o[e] *= alpha;
                m = s;
            }
            const float p = expf(s - m);
            l += p;
            for (int e = 0; e < kSub; ++e) o[e] += p * Vs[j][part * kSub + e];
        }
    }
    if (!valid) return;
    float* orow = (float*)out.data + (int64_t)b * out.sB + (int64_t)row * out.sS + (int64_t)h * out.sH + part * kSub;
    float* lrow = lse.data + (int64_t)b * lse.sB + (int64_t)h * lse.sH + row;
    if (l == 0.f) {  // no valid key in the chunk: the partial is the merge identity
        if (!merge) {
            for (int e = 0; e < kSub; ++e) orow[e] = 0.f;
            if (part == 0) *lrow = -INFINITY;
        }
        return;
    }
    const float lse_c = m + logf(l);
    const float inv_l = 1.f / l;
    if (!merge) {
        for (int e = 0; e < kSub; ++e) orow[e] = o[e] * inv_l;
        if (part == 0) *lrow = lse_c;
    } else {
        const float la = *lrow;
        const float mm = fmaxf(la, lse_c);
        const float ea = expf(la - mm), ec = expf(lse_c - mm);
        const float sum = ea + ec;
        const float wa = ea / sum, wc = ec / sum * inv_l;
        for (int e = 0; e < kSub; ++e) orow[e] = (wa == 0.f ? 0.f : wa * orow[e]) + wc * o[e];
        // the T lanes of this row are adjacent in one wavefront: all have read lse_acc
        if (part == 0) *lrow = mm + logf(sum);
    }
}

// ---------------------------------------------------------------- backward: dQ of a chunk
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dq_f32_kernel(ra_tensor q, ra_tensor k, ra_tensor v, ra_tensor dout,
                                                              ra_lse lse, ra_lse delta, KeyMask km, float scale,
                                                              ra_tensor dq) {
    constexpr int T = D / kSub;
    constexpr int RowsPerBlock = kThreads / T;
    __shared__ float Ks[kTile][D];
    __shared__ float Vs[kTile][D];
    const int b = blockIdx.z, h = blockIdx.y;
    const int g = h / (q.H / k.H);
    const int part = threadIdx.x % T;
    const int row = blockIdx.x * RowsPerBlock + threadIdx.x / T;
    const bool valid = row < q.S;
    float qr[kSub], dor[kSub], acc[kSub];
    for (int j = 0; j < kSub; ++j) {
        qr[j] = valid ? rowp(q, b, row, h)[part * kSub + j] : 0.f;
        dor[j] = valid ? rowp(dout, b, row, h)[part * kSub + j] : 0.f;
        acc[j] = 0.f;
    }
    const float lse_r = valid ? lse.data[(int64_t)b * lse.sB + (int64_t)h * lse.sH + row] : 0.f;
    const float dl_r = valid ? delta.data[(int64_t)b * delta.sB + (int64_t)h * delta.sH + row] : 0.f;
    for (int n0 = 0; n0 < k.S; n0 += kTile) {
        __syncthreads();
        stage_rows<D>(Ks, k, b, g, n0, k.S);
        stage_rows<D>(Vs, v, b, g, n0, k.S);
        __syncthreads();
        const int nk = min(kTile, k.S - n0);
        for (int j = 0; j < nk; ++j) {
            if (!key_on(km, b, n0 + j)) continue;
            float s = 0.f, dp = 0.f;
            for (int e = 0; e < kSub; ++e) {
                s += qr[e] * Ks[j][part * kSub + e];
                dp += dor[e] * Vs[j][part * kSub + e];
            }
            s = group_sum<T>(s) * scale;
            dp = group_sum<T>(dp);
            const float p = expf(s - lse_r);
            const float ds = p * (dp - dl_r);
            for (int e = 0; e < kSub; ++e) acc[e] += ds * Ks[j][part * kSub + e];
        }
    }
    if (!valid) return;
    float* drow = (float*)dq.data + (int64_t)b * dq.sB + (int64_t)row * dq.sS + (int64_t)h * dq.sH + part * kSub;
    for (int e = 0; e < kSub; ++e) drow[e] += scale * acc[e];
}

// ---------------------------------------------------------------- backward: dK, dV of a chunk
// A key row is owned by T lanes; the block sweeps every query row of every query
// head of the key's group, staged through LDS.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_f32_kernel(ra_tensor q, ra_tensor k, ra_tensor v, ra_tensor dout,
                                                                ra_lse lse, ra_lse delta, KeyMask km, float scale,
                                                                ra_tensor dk, ra_tensor dv) {
    constexpr int T = D / kSub;
    constexpr int RowsPerBlock = kThreads / T;
    __shared__ float Qs[kTile][D];
    __shared__ float Os[kTile][D];
    __shared__ float Ls[kTile], Ds[kTile];
    const int b = blockIdx.z, g = blockIdx.y;
    const int G = q.H / k.H;
    const int part = threadIdx.x % T;
    const int key = blockIdx.x * RowsPerBlock + threadIdx.x / T;
    const bool valid = key < k.S;
    float kr[kSub], vr[kSub], dka[kSub], dva[kSub];
    for (int j = 0; j < kSub; ++j) {
        kr[j] = valid ? rowp(k, b, key, g)[part * kSub + j] : 0.f;
        vr[j] = valid ? rowp(v, b, key, g)[part * kSub + j] : 0.f;
        dka[j] = 0.f;
        dva[j] = 0.f;
    }
    for (int hh = 0; hh < G; ++hh) {
        const int h = g * G + hh;
        for (int r0 = 0; r0 < q.S; r0 += kTile) {
            __syncthreads();
            stage_rows<D>(Qs, q, b, h, r0, q.S);
            stage_rows<D>(Os, dout, b, h, r0, q.S);
            for (int i = threadIdx.x; i < kTile; i += kThreads) {
                const bool in = r0 + i < q.S;
                Ls[i] = in ? lse.data[(int64_t)b * lse.sB + (int64_t)h * lse.sH + r0 + i] : 0.f;
                Ds[i] = in ? delta.data[(int64_t)b * delta.sB + (int64_t)h * delta.sH + r0 + i] : 0.f;
            }
            __syncthreads();
            const int nr = min(kTile, q.S - r0);
            for (int i = 0; i < nr; ++i) {
                float s = 0.f, dp = 0.f;
                for (int e = 0; e < kSub; ++e) {
                    s += Qs[i][part * kSub + e] * kr[e];
                    dp += Os[i][part * kSub + e] * vr[e];
                }
                s = group_sum<T>(s) * scale;
                dp = group_sum<T>(dp);
                const float p = expf(s - Ls[i]);
                const float ds = p * (dp - Ds[i]);
                for (int e = 0; e < kSub; ++e) {
                    dva[e] += p * Os[i][part * kSub + e];
                    dka[e] += ds * Qs[i][part * kSub + e];
                }
            }
        }
    }
    if (!valid || !key_on(km, b, key)) return;  // a masked key gets no dK/dV
    float* kd = (float*)dk.data + (int64_t)b * dk.sB + (int64_t)key * dk.sS + (int64_t)g * dk.sH + part * kSub;
    float* vd = (float*)dv.data + (int64_t)b * dv.sB + (int64_t)key * dv.sS + (int64_t)g * dv.sH + part * kSub;
    for (int e = 0; e < kSub; ++e) {
        kd[e] += scale * dka[e];
        vd[e] += dva[e];
    }
}

}  // namespace

hipError_t launch_fwd_chunk_f32(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const KeyMask& km,
                                float scale, const ra_tensor& out, const ra_lse& lse, int merge, hipStream_t s) {
    if (q.S == 0) return hipSuccess;
    const int T = q.D / kSub;
    dim3 grid((q.S + kThreads / T - 1) / (kThreads / T), q.H, q.B);
    if (q.D == 64)
        fwd_f32_kernel<64><<<grid, kThreads, 0, s>>>(q, k, v, km, scale, out, lse, merge);
    else
        fwd_f32_kernel<128><<<grid, kThreads, 0, s>>>(q, k, v, km, scale, out, lse, merge);
    return hipGetLastError();
}

hipError_t launch_bwd_dq_f32(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const ra_tensor& dout,
                             const ra_lse& lse, const ra_lse& delta, const KeyMask& km, float scale,
                             const ra_tensor& dq_acc, hipStream_t s) {
    if (q.S == 0 || k.S == 0) return hipSuccess;
    const int rpb = kThreads / (q.D / kSub);
    dim3 g((q.S + rpb - 1) / rpb, q.H, q.B);
    if (q.D == 64) bwd_dq_f32_kernel<64><<<g, kThreads, 0, s>>>(q, k, v, dout, lse, delta, km, scale, dq_acc);
    else bwd_dq_f32_kernel<128><<<g, kThreads, 0, s>>>(q, k, v, dout, lse, delta, km, scale, dq_acc);
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv_f32(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const ra_tensor& dout,
                               const ra_lse& lse, const ra_lse& delta, const KeyMask& km, float scale,
                               const ra_tensor& dk_acc, const ra_tensor& dv_acc, hipStream_t s) {
    if (q.S == 0 || k.S == 0) return hipSuccess;
    const int rpb = kThreads / (q.D / kSub);
    dim3 g((k.S + rpb - 1) / rpb, k.H, k.B);
    if (q.D == 64) bwd_dkdv_f32_kernel<64><<<g, kThreads, 0, s>>>(q, k, v, dout, lse, delta, km, scale, dk_acc, dv_acc);
    else bwd_dkdv_f32_kernel<128><<<g, kThreads, 0, s>>>(q, k, v, dout, lse, delta, km, scale, dk_acc, dv_acc);
    return hipGetLastError();
}

}  // namespace ra
