// kda_state_io.hip -- zero / copy / gather / scatter of KDA state pools with
// fp32 <-> bf16 conversion.  Pools are [slots, H, 128, 128] with each slot's
// heads stored one after another ("Kimi K3 -- Training and Infrastructure
// Notes", section 4.5: head-by-head contiguous states; a prefix-cache hit copies
// a read-only snapshot into the request's private state, new checkpoints go to
// fresh slots).  Pure streaming copies: 16-byte (fp32) or 8-byte (bf16) vector
// accesses, one grid row of workgroups per state.
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

template <class Src, class Dst>
__global__ __launch_bounds__(256) void state_io_kernel(int op, const Src *__restrict__ src,
                                                       int32_t src_slots, Dst *__restrict__ dst,
                                                       int32_t dst_slots,
                                                       const int32_t *__restrict__ indices,
                                                       int64_t elems, int32_t parts) {
  // blockIdx.x = state i * parts + part; `parts` workgroups share one state.
  const int64_t i = blockIdx.x / parts;
  const int part = (int)(blockIdx.x - i * parts);
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
  const int64_t n4 = elems / 4;
  const SV *sp = reinterpret_cast<const SV *>(src + s_src * elems);
  DV *dp = reinterpret_cast<DV *>(dst + s_dst * elems);
  for (int64_t e = (int64_t)part * blockDim.x + threadIdx.x; e < n4;
       e += (int64_t)parts * blockDim.x) {
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (op != KDA_STATE_ZERO) x = Vec4<Src>::to(sp[e]);
    dp[e] = Vec4<Dst>::from(x);
  }
}

template <class Src, class Dst>
hipError_t launch_typed(kda_state_op op, const void *src, int32_t src_slots, void *dst,
                        int32_t dst_slots, const int32_t *indices, int32_t count,
                        int64_t elems, hipStream_t stream) {
  const int64_t n4 = elems / 4;
  int64_t parts = (n4 + 255) / 256;
  if (parts > 64) parts = 64;
  hipLaunchKernelGGL((state_io_kernel<Src, Dst>), dim3((unsigned)(parts * count)), dim3(256),
                     0, stream, (int)op, (const Src *)src, src_slots, (Dst *)dst, dst_slots,
                     indices, elems, (int32_t)parts);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_state_io(kda_state_op op, const void *src, kda_dtype src_dtype,
                           int32_t src_slots, void *dst, kda_dtype dst_dtype,
                           int32_t dst_slots, const int32_t *indices, int32_t count,
                           int64_t elems_per_state, hipStream_t stream) {
  if (count == 0) return hipSuccess;
  if (op == KDA_STATE_ZERO) src_dtype = dst_dtype;  // src unused
  if (src_dtype == KDA_F32 && dst_dtype == KDA_F32)
    return launch_typed<float, float>(op, src, src_slots, dst, dst_slots, indices, count,
                                      elems_per_state, stream);
  if (src_dtype == KDA_F32 && dst_dtype == KDA_BF16)
    return launch_typed<float, bf16>(op, src, src_slots, dst, dst_slots, indices, count,
                                     elems_per_state, stream);
  if (src_dtype == KDA_BF16 && dst_dtype == KDA_F32)
    return launch_typed<bf16, float>(op, src, src_slots, dst, dst_slots, indices, count,
                                     elems_per_state, stream);
  return launch_typed<bf16, bf16>(op, src, src_slots, dst, dst_slots, indices, count,
                                  elems_per_state, stream);
}

}  // namespace kda
