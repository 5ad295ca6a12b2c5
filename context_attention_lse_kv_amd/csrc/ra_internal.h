// Internal interface between the C-ABI layer (ra_abi.cpp) and the kernel
// launchers (*.hip).  Descriptors are passed to kernels by value.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/ra.h"

namespace ra {

// Tile geometry of the bf16 MFMA kernels (also used by host-side sizing).
constexpr int kFwdRowsPerWave = 32;
constexpr int kFwdWaves = 4;
constexpr int kFwdBlockM = kFwdRowsPerWave * kFwdWaves;  // query rows per workgroup
constexpr int kFwdBlockN = 64;                            // keys per LDS tile
constexpr int kBwdKeysPerWave = 32;
constexpr int kBwdWaves = 4;
constexpr int kBwdBlockN = kBwdKeysPerWave * kBwdWaves;  // keys per workgroup
constexpr int kBwdBlockM = 64;                            // query rows per LDS tile

// dS workspace of the bf16 backward (written by the dK/dV kernel, read by the dQ pass):
// one 4 KiB block (64 query rows x 32 keys, bf16) per (batch, query head, 32-key group,
// 64-row query tile); key groups are counted up to whole 128-key workgroup tiles.
constexpr int64_t kDsBlockBytes = 4096;
inline int ds_query_tiles(int Sq) { return (Sq + 63) / 64; }
inline int ds_key_groups(int Sk) { return 4 * ((Sk + kBwdBlockN - 1) / kBwdBlockN); }
inline int64_t ds_bytes(int B, int Hq, int Sq, int Sk) {
    return (int64_t)B * Hq * ds_query_tiles(Sq) * ds_key_groups(Sk) * kDsBlockBytes;
}
// the dQ pass over stored dS: kDqsWaves wavefronts, one 64-row query tile each, per workgroup
constexpr int kDqsWaves = 8;
constexpr int kDqsMaxChunks = 8;  // chunks one dQ pass can sweep
inline int64_t dqs_workgroups(int B, int Hq, int Sq) {
    return (int64_t)B * Hq * ((ds_query_tiles(Sq) + kDqsWaves - 1) / kDqsWaves);
}
constexpr int kMaxRanks = 16;  // exchange fan-out limit (kernel argument table)

// Size of the per-GPU device array that ra_ring_fwd_noalloc uses as its workspace (the
// fp32 running output of a bf16 sweep: 16 Mi elements, e.g. 4096 query rows x 32 heads x
// 128).  scratch_region returns its device address on the current device (looked up
// once per device) and its size.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t scratch_region(void** ptr, size_t* bytes);

// Key mask of one chunk as the kernels see it: data[b * sB + key] != 0 means the key
// takes part; data == nullptr means every key does.
struct KeyMask {
    const uint8_t* data;
    int64_t sB;
};

// Unsigned 32-bit division by an invariant d >= 1 as a multiply-high and two shifts
// (Granlund and Montgomery, "Division by invariant integers using multiplication", the
// round-up method): q = (t + ((n - t) >> s1)) >> s2 with t = mulhi(m, n).
struct UDiv {
    uint32_t m;
    uint16_t s1, s2;
};

struct PermuteTable {
    int32_t n_in, n_out, dir, elem_bytes;
    ra_tensor in[kMaxRanks];
    ra_tensor out[kMaxRanks];
    int32_t off[kMaxRanks + 1];  // seq offsets (dir 0: of inputs; dir 1: of outputs)
    int32_t hoff[kMaxRanks + 1]; // head offsets (dir 0: of outputs; dir 1: of inputs)
    // filled by launch_permute: division by the 16-byte vectors per row, and per rank by the
    // head count (dh) and row count (dl) of the (output, input) sub-copies
    UDiv dv, dh[kMaxRanks], dl[kMaxRanks];
};

// All launchers enqueue on `s` and return hipGetLastError() of the launch.
// Shapes have been validated by the caller.
// out16 (bf16, shape of q): when given, the step is the sweep's last and its (merged)
// output is written there in bf16 instead of to out; lse is written as usual.
hipError_t launch_fwd_chunk_bf16(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const KeyMask& km,
                                 float scale, const ra_tensor& out, const ra_lse& lse, int merge, hipStream_t s,
                                 const ra_tensor* out16 = nullptr);
hipError_t launch_fwd_chunk_f32(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const KeyMask& km,
                                float scale, const ra_tensor& out, const ra_lse& lse, int merge, hipStream_t s);
// Backward chunk step, split: add this chunk's contribution to dk_acc/dv_acc, or to
// dq_acc (all fp32).
// ds: dS workspace of ds_bytes(q.B, q.H, q.S, k.S) bytes that receives this chunk
// step's dS (bf16, zero for keys outside the chunk or masked), or null.  dk_out/dv_out
// (bf16, the chunk's rows): when given, the launch's dK/dV are final and written there
// instead of being added to dk_acc/dv_acc (which are then not touched).
hipError_t launch_bwd_dkdv_bf16(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const ra_tensor& dout,
                                const ra_lse& lse, const ra_lse& delta, const KeyMask& km, float scale,
                                const ra_tensor& dk_acc, const ra_tensor& dv_acc, void* ds, hipStream_t s,
                                const ra_tensor* dk_out = nullptr, const ra_tensor* dv_out = nullptr);
// dq_acc += scale dS K from the dS workspace written by launch_bwd_dkdv_bf16 for the same
// q rows and chunk k.  dq_read = false: dq_acc counts as zero (it is only written);
// dq_out (bf16): when given, the sum is final and written there instead of dq_acc.
// km: the chunk's key mask the dS was stored under (its masked keys hold zero dS), or
// null; with it the pass skips the key tiles after the last valid key.  more: up to
// kDqsMaxChunks - 1 further chunks (rows of the same k tensor, same q rows) whose dS is
// swept after the first one's in the same pass, so that dq_acc is read and written once
// for all of them.
struct DqsChunk {
    ra_tensor k;
    const void* ds;
    const KeyMask* km;
};
hipError_t launch_bwd_dqs_bf16(const ra_tensor& q, const ra_tensor& k, const void* ds, float scale,
                               const ra_tensor& dq_acc, hipStream_t s, bool dq_read = true,
                               const ra_tensor* dq_out = nullptr, const KeyMask* km = nullptr,
                               const DqsChunk* more = nullptr, int n_more = 0);
hipError_t launch_bwd_dq_bf16(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const ra_tensor& dout,
                              const ra_lse& lse, const ra_lse& delta, const KeyMask& km, float scale,
                              const ra_tensor& dq_acc, hipStream_t s);
hipError_t launch_bwd_dkdv_f32(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const ra_tensor& dout,
                               const ra_lse& lse, const ra_lse& delta, const KeyMask& km, float scale,
                               const ra_tensor& dk_acc, const ra_tensor& dv_acc, hipStream_t s);
hipError_t launch_bwd_dq_f32(const ra_tensor& q, const ra_tensor& k, const ra_tensor& v, const ra_tensor& dout,
                             const ra_lse& lse, const ra_lse& delta, const KeyMask& km, float scale,
                             const ra_tensor& dq_acc, hipStream_t s);
hipError_t launch_merge_lse(const ra_tensor& out_acc, const ra_lse& lse_acc, const ra_tensor& out_part,
                            const ra_lse& lse_part, hipStream_t s);
hipError_t launch_bwd_delta(const ra_tensor& out, const ra_tensor& dout, const ra_lse& delta, hipStream_t s);
hipError_t launch_cast_f32_to_bf16(const ra_tensor& src, const ra_tensor& dst, hipStream_t s);
hipError_t launch_zero_f32(const ra_tensor& t, hipStream_t s);
hipError_t launch_fill_rows(const ra_lse& t, float value, hipStream_t s);
hipError_t launch_permute(const PermuteTable& tab, hipStream_t s);

}  // namespace ra
