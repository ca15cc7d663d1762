// kernels.h - host-side launchers of the gfx950 kernels (one per .hip file group).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <tuple>
#include <utility>

#include "device.h"

namespace hsa {

// Optional start/stop events, recorded by the dispatch itself (hipExtLaunchKernel):
// their interval is the kernel's own execution, with no launch gap around it.
// `fired` is set when the events were attached to a launch.
struct LaunchEv {
  hipEvent_t a = nullptr, b = nullptr;
  bool* fired = nullptr;
};

template <class... KArgs, class... Args>
inline hipError_t launch_k(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t st,
                           const LaunchEv& ev, Args&&... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  std::tuple<KArgs...> t{std::forward<Args>(args)...};
  return std::apply(
      [&](auto&... a) {
        void* argv[] = {static_cast<void*>(&a)...};
        const hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block,
                                                argv, 0, st, ev.a, ev.b, 0);
        if (e == hipSuccess && ev.a && ev.fired) *ev.fired = true;
        return e;
      },
      t);
}

// append_seal.hip
hipError_t launch_decode_append(const Pools& P, const ReqBatch& B, const void* kin, const void* vin,
                                const float* iin, float* part, hipStream_t st,
                 const LaunchEv& ev = LaunchEv{});
// Fold the kSealSplit HCA partials of each block sealed by launch_decode_append.
hipError_t launch_seal_merge(const Pools& P, const ReqBatch& B, const float* part, hipStream_t st,
                 const LaunchEv& ev = LaunchEv{});
hipError_t launch_bulk_seal(const Pools& P, const SealDesc* seals, int64_t n_seals, const void* kin,
                            const void* vin, const float* iin, hipStream_t st,
                 const LaunchEv& ev = LaunchEv{});
hipError_t launch_bulk_write(const Pools& P, const WriteDesc* w, int32_t n_req, int64_t total,
                             const void* kin, const void* vin, const float* iin, hipStream_t st,
                 const LaunchEv& ev = LaunchEv{});

// indexer_topk.hip
// Scores of every sealed C4 entry of the batch's requests: scores[i * ld + j].
hipError_t launch_score(const Pools& P, const ReqBatch& B, int64_t total_blocks, const float* q_idx,
                        float* scores, int64_t ld, hipStream_t st,
                 const LaunchEv& ev = LaunchEv{});
// Top-k of each request's scores (one workgroup per request or per slice of a long
// row, then a second launch for sliced rows), in ascending ordinal order, or by
// (score desc, ordinal asc) when `sorted`.
hipError_t launch_select(const ReqBatch& B, const SelPlan& SP, int32_t k, int32_t sorted,
                         const float* scores, int64_t ld, int32_t* idx_out, float* score_out,
                         hipStream_t st, const LaunchEv& ev = LaunchEv{});

// Per-row FP8 storage (the C4 entry quantisation) of n_rows rows of 128 floats.
hipError_t launch_fp8_rows(const float* x, int64_t n_rows, uint8_t* codes, float* scales,
                           hipStream_t st);
// Eager C4: recompute the listed open-block entries from the states' rings.
hipError_t launch_open_c4(const Pools& P, const OpenDesc* d, int32_t n, hipStream_t st);
// Batched copy of n segments (total chunks of 64 KiB), staged on the device.
hipError_t launch_copy_segs(const CopySeg* d, int32_t n, int64_t total, hipStream_t st);
// Table rows of states attached to a prefix (block ids staged on the device).
hipError_t launch_attach_rows(const Pools& P, const AttachDesc* d, int32_t n, const int32_t* ids,
                              hipStream_t st);
// Per-key MXFP4 storage (the sealed indexer key quantisation) of n_rows keys of 256 floats.
hipError_t launch_mx4_rows(const float* x, int64_t n_rows, uint8_t* codes, uint8_t* scales,
                           hipStream_t st);

// attend.hip
// Keys of request i: min(len, n_win) SWA + nb HCA + min(k, 32 nb) C4 slots, cut in
// chunks of `chunk` keys (a multiple of 16); one workgroup per chunk writes an
// unnormalised partial, or out[i] directly when request i is one chunk.
hipError_t launch_attend(const Pools& P, const ReqBatch& B, int64_t total_chunks, int32_t chunk,
                         const void* q, const int32_t* topk, int32_t k, float* part_acc,
                         float* part_ml, float* out, hipStream_t st,
                 const LaunchEv& ev = LaunchEv{});
// Merge the chunk partials of every request with two or more chunks into out.
hipError_t launch_merge(const Pools& P, const ReqBatch& B, int32_t chunk, int32_t k,
                        const float* part_acc, const float* part_ml, float* out, hipStream_t st,
                 const LaunchEv& ev = LaunchEv{});

// step.hip: the decode step in three or four launches (see step.hip for what each
// does; launch_step2b and launch_step3 enqueue nothing in the three-launch form).
hipError_t launch_step1(const Pools& P, const ReqBatch& B, const StepArgs& S, hipStream_t st,
                 const LaunchEv& ev = LaunchEv{});
hipError_t launch_step2(const Pools& P, const ReqBatch& B, const StepArgs& S, hipStream_t st,
                 const LaunchEv& ev = LaunchEv{});
hipError_t launch_step2b(const Pools& P, const ReqBatch& B, const StepArgs& S, hipStream_t st,
                 const LaunchEv& ev = LaunchEv{});
hipError_t launch_step3(const Pools& P, const ReqBatch& B, const StepArgs& S, hipStream_t st,
                 const LaunchEv& ev = LaunchEv{});
hipError_t launch_step4(const Pools& P, const ReqBatch& B, const StepArgs& S, hipStream_t st,
                 const LaunchEv& ev = LaunchEv{});

}  // namespace hsa
