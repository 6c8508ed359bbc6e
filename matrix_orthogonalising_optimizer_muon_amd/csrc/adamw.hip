// AdamW step for the parameters Muon does not update (embeddings, biases, norm weights):
// MuonX article, section 2 -- AdamW adjusts each element from running averages of the
// gradient and of its square; the hidden 2-D weights go to Muon, the rest to AdamW.
//
// One launch covers up to kAdamChunk tensors (their pointers travel in the kernel
// arguments); each 256-thread workgroup updates 2048 consecutive elements of one tensor,
// 8 per thread with 16-byte accesses where alignment allows. The step is HBM-bound:
// per element W read + write, G read, m and v (fp32) read + write.
#include "internal.hpp"

namespace muon {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 8;
constexpr int kPerBlock = kThreads * kPerThread;

__device__ __forceinline__ float bf16_to_f32(unsigned short h) {
  return __uint_as_float(static_cast<unsigned int>(h) << 16);
}
__device__ __forceinline__ unsigned short f32_to_bf16(float f) {
  unsigned int u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<unsigned short>(u >> 16);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// 16-byte load; NT marks it non-temporal. Only G, read once and never written, is loaded
// that way: non-temporal loads of W, m and v, which the step writes back, measured slower
// (7B non-matrix set on one MI355X: 6.1 ms against 5.5 ms), the G-only form faster (5.43 ms).
template <bool NT>
__device__ __forceinline__ u32x4 ld16(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  else return *static_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *static_cast<u32x4*>(p) = v; }

template <bool NT = false>
__device__ __forceinline__ void load8(const void* p, int64_t i, int bf16, float (&v)[8]) {
  if (bf16) {
    const u32x4 w = ld16<NT>(static_cast<const unsigned short*>(p) + i);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(w[q] << 16);
      v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
    }
  } else {
    const float* f = static_cast<const float*>(p) + i;
    const u32x4 a = ld16<NT>(f), b = ld16<NT>(f + 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = __uint_as_float(a[q]);
      v[4 + q] = __uint_as_float(b[q]);
    }
  }
}
__device__ __forceinline__ void store8(void* p, int64_t i, int bf16, const float (&v)[8]) {
  if (bf16) {
    u32x4 w;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = f32_to_bf16(v[2 * q]) | (static_cast<unsigned int>(f32_to_bf16(v[2 * q + 1])) << 16);
    st16(static_cast<unsigned short*>(p) + i, w);
  } else {
    float* f = static_cast<float*>(p) + i;
    st16(f, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
    st16(f + 4, u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])});
  }
}
__device__ __forceinline__ float load1(const void* p, int64_t i, int bf16) {
  return bf16 ? bf16_to_f32(static_cast<const unsigned short*>(p)[i]) : static_cast<const float*>(p)[i];
}
__device__ __forceinline__ void store1(void* p, int64_t i, int bf16, float v) {
  if (bf16) static_cast<unsigned short*>(p)[i] = f32_to_bf16(v);
  else static_cast<float*>(p)[i] = v;
}

__global__ __launch_bounds__(kThreads) void adamw_kernel(const AdamChunk c) {
  // Which tensor this workgroup serves: the last one whose first block is <= blockIdx.x.
  const int64_t b = blockIdx.x;
  int t = 0;
  for (int i = 1; i < c.n; ++i)
    if (c.t[i].block0 <= b) t = i;
  const AdamTensor& T = c.t[t];
  const int64_t e0 = (b - T.block0) * kPerBlock + static_cast<int64_t>(threadIdx.x) * kPerThread;
  if (e0 >= T.numel) return;

  const float decay = 1.0f - c.lr * c.wd;
  const float step = c.lr / c.bc1;
  auto update = [&](float& w, float g, float& m, float& v) {
    w *= decay;
    m = c.b1 * m + (1.0f - c.b1) * g;
    v = c.b2 * v + (1.0f - c.b2) * g * g;
    w -= step * m / (sqrtf(v) / c.bc2s + c.eps);
  };

  if (T.vec && e0 + kPerThread <= T.numel) {
    float w[8], g[8], m[8], v[8];
    load8(T.W, e0, c.w_bf16, w);
    load8<true>(T.G, e0, c.g_bf16, g);
    load8(T.m, e0, 0, m);
    load8(T.v, e0, 0, v);
#pragma unroll
    for (int k = 0; k < 8; ++k) update(w[k], g[k], m[k], v[k]);
    store8(T.W, e0, c.w_bf16, w);
    store8(T.m, e0, 0, m);
    store8(T.v, e0, 0, v);
  } else {
    for (int k = 0; k < kPerThread; ++k) {
      const int64_t e = e0 + k;
      if (e >= T.numel) break;
      float w = load1(T.W, e, c.w_bf16), m = T.m[e], v = T.v[e];
      update(w, load1(T.G, e, c.g_bf16), m, v);
      store1(T.W, e, c.w_bf16, w);
      T.m[e] = m;
      T.v[e] = v;
    }
  }
}

}  // namespace

int64_t adam_blocks(int64_t numel) { return (numel + kPerBlock - 1) / kPerBlock; }

hipError_t launch_adamw(const AdamChunk& c, int64_t blocks, hipStream_t st) {
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(adamw_kernel, dim3(static_cast<unsigned int>(blocks)), dim3(kThreads), 0, st, c);
  return hipGetLastError();
}

}  // namespace muon
