// kda_state_io.hip -- zero / copy / gather / scatter of KDA state pools with
// fp32 <-> bf16 conversion.  Pools are [slots, H, 128, 128] with each slot's
// heads stored one after another ("Kimi K3 -- Training and Infrastructure
// Notes", section 4.5: head-by-head contiguous states; a prefix-cache hit copies
// a read-only snapshot into the request's private state, new checkpoints go to
// fresh slots).  Pure streaming copies: 16-byte (fp32) or 8-byte (bf16) vector
// accesses, one workgroup per head of a state.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

template <class T> struct Vec4;
template <> struct Vec4<float> {
  typedef f32x4 type;
  static __device__ __forceinline__ f32x4 to(const type &x) { return x; }
  static __device__ __forceinline__ type from(const f32x4 &x) { return x; }
};
template <> struct Vec4<bf16> {
  typedef bf16x4 type;
  static __device__ __forceinline__ f32x4 to(const type &x) {
    f32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (float)x[i];
    return r;
  }
  static __device__ __forceinline__ type from(const f32x4 &x) {
    type r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (bf16)x[i];
    return r;
  }
};

// One 512-thread workgroup per head-state (128 x 128 elements): every thread
// loads its 8 vectors of 4 elements, then stores them, with non-temporal hints
// (each byte is streamed once).  Measured against other shapes of the same copy
// (512 x 96 fp32 head-states, 3.2 GB each way): one workgroup per head, loads
// before stores, non-temporal: 0.69 of the HBM peak; a grid-stride loop with one
// vector per thread and iteration: 0.60-0.64.
constexpr int kIoThreads = 512;
constexpr int kIoVecs = KDA_HEAD_DIM * KDA_HEAD_DIM / 4 / kIoThreads;  // 8 per thread

template <class Src, class Dst>
__global__ __launch_bounds__(kIoThreads) void state_io_kernel(int op, const Src *__restrict__ src,
                                                              int32_t src_slots, Dst *__restrict__ dst,
                                                              int32_t dst_slots,
                                                              const int32_t *__restrict__ indices,
                                                              int32_t num_heads) {
  // blockIdx.x = position i * num_heads + head
  const int64_t i = blockIdx.x / num_heads;
  const int head = (int)(blockIdx.x - i * num_heads);
  int64_t s_src = i, s_dst = i;
  if (op == KDA_STATE_ZERO) {
    s_dst = indices ? indices[i] : i;
  } else if (op == KDA_STATE_GATHER) {
    s_src = indices[i];
  } else if (op == KDA_STATE_SCATTER) {
    s_dst = indices[i];
  }
  if (s_dst < 0 || s_dst >= dst_slots) return;
  if (op != KDA_STATE_ZERO && (s_src < 0 || s_src >= src_slots)) return;
  typedef typename Vec4<Src>::type SV;
  typedef typename Vec4<Dst>::type DV;
  constexpr int64_t kHeadVecs = KDA_HEAD_DIM * KDA_HEAD_DIM / 4;
  const SV *sp = reinterpret_cast<const SV *>(src) + (s_src * num_heads + head) * kHeadVecs;
  DV *dp = reinterpret_cast<DV *>(dst) + (s_dst * num_heads + head) * kHeadVecs;
  f32x4 x[kIoVecs];
#pragma unroll
  for (int u = 0; u < kIoVecs; ++u)
    x[u] = op == KDA_STATE_ZERO ? f32x4{0.f, 0.f, 0.f, 0.f}
                                : Vec4<Src>::to(__builtin_nontemporal_load(sp + u * kIoThreads + threadIdx.x));
#pragma unroll
  for (int u = 0; u < kIoVecs; ++u)
    __builtin_nontemporal_store(Vec4<Dst>::from(x[u]), dp + u * kIoThreads + threadIdx.x);
}

template <class Src, class Dst>
hipError_t launch_typed(kda_state_op op, const void *src, int32_t src_slots, void *dst,
                        int32_t dst_slots, const int32_t *indices, int32_t count,
                        int32_t num_heads, hipStream_t stream) {
  hipLaunchKernelGGL((state_io_kernel<Src, Dst>), dim3((unsigned)((int64_t)count * num_heads)),
                     dim3(kIoThreads), 0, stream, (int)op, (const Src *)src, src_slots, (Dst *)dst,
                     dst_slots, indices, num_heads);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_state_io(kda_state_op op, const void *src, kda_dtype src_dtype,
                           int32_t src_slots, void *dst, kda_dtype dst_dtype,
                           int32_t dst_slots, const int32_t *indices, int32_t count,
                           int32_t num_heads, hipStream_t stream) {
  if (count == 0) return hipSuccess;
  if (op == KDA_STATE_ZERO) src_dtype = dst_dtype;  // src unused
  if (src_dtype == KDA_F32 && dst_dtype == KDA_F32)
    return launch_typed<float, float>(op, src, src_slots, dst, dst_slots, indices, count,
                                      num_heads, stream);
  if (src_dtype == KDA_F32 && dst_dtype == KDA_BF16)
    return launch_typed<float, bf16>(op, src, src_slots, dst, dst_slots, indices, count,
                                     num_heads, stream);
  if (src_dtype == KDA_BF16 && dst_dtype == KDA_F32)
    return launch_typed<bf16, float>(op, src, src_slots, dst, dst_slots, indices, count,
                                     num_heads, stream);
  return launch_typed<bf16, bf16>(op, src, src_slots, dst, dst_slots, indices, count,
                                  num_heads, stream);
}

}  // namespace kda
