// kv_compress: softmax-weighted fold of m consecutive tokens into one shared
// K=V entry, rotated at the position of the group's first token
// (V4 page, section 2.1 compressor; section 3.1.2 rolling residual;
// section 3.2.1 RoPE before cache insertion).
//
// HBM-bound stream: each thread owns 8 consecutive dims (one 16-byte bf16
// load per token) so a row of d dims is read by d/8 adjacent lanes in one
// coalesced sweep.  Small m: a row-group of d/8 threads folds whole entries on
// its own.  Large m: the 256 threads of a block share one entry (or, when
// there are few entries, as in a decode step, one 64-dim slice of it), each
// row-group folding a strided subset of its tokens, reduced through LDS.
#include "hca_common.h"
#include "hca_internal.h"

namespace hca {

constexpr int kCompressThreads = 256;
constexpr int kSmallM = 16;

__device__ __forceinline__ void load_bf16x8(const uint16_t* p, float v[8]) {
  const u32x4 raw = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = u2f(raw[i] << 16);
    v[2 * i + 1] = u2f(raw[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ void rope_store8(float* dst, const float acc[8], double pos, const double inv[4]) {
  float o[8];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    float c, s;
    rope_cs(pos, inv[p], c, s);
    o[2 * p] = acc[2 * p] * c - acc[2 * p + 1] * s;
    o[2 * p + 1] = acc[2 * p] * s + acc[2 * p + 1] * c;
  }
  f32x4* d4 = reinterpret_cast<f32x4*>(dst);
  d4[0] = f32x4{o[0], o[1], o[2], o[3]};
  d4[1] = f32x4{o[4], o[5], o[6], o[7]};
}

__global__ __launch_bounds__(kCompressThreads) void compress_kernel(CompressArgs a) {
  const int TD = a.d >> 3;              // threads across the dims of a row
  const int RP = kCompressThreads / TD; // row groups
  const int li = threadIdx.x % TD;
  const int gi = threadIdx.x / TD;
  const bool active = gi < RP;
  const int b = blockIdx.y;
  const int n = clampi(a.ntok[b], 0, a.max_ntok);
  const int m = a.m;
  const int N = (n + m - 1) / m;
  const int p0 = a.pos0[b];
  const uint16_t* xb = a.x + (int64_t)b * a.xs + li * 8;
  const float* zb = a.z + (int64_t)b * a.zs;
  float* ob = a.out + (int64_t)b * a.os + li * 8;

  double inv[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) inv[p] = rope_inv_freq(li * 4 + p, a.d, a.theta);

  if (m <= kSmallM) {
    if (!active) return;
    for (int j = blockIdx.x * RP + gi; j < N; j += gridDim.x * RP) {
      const int t0 = j * m;
      const int r = min(m, n - t0);
      float mx = -INFINITY;
      for (int i = 0; i < r; ++i) mx = fmaxf(mx, zb[t0 + i] + a.beta[i]);
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      float tot = 0.0f;
      for (int i = 0; i < r; ++i) {
        const float e = expf(zb[t0 + i] + a.beta[i] - mx);
        tot += e;
        float v[8];
        load_bf16x8(xb + (int64_t)(t0 + i) * a.d, v);
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = fmaf(e, v[c], acc[c]);
      }
      const float inv_tot = 1.0f / tot;
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] *= inv_tot;
      rope_store8(ob + (int64_t)j * a.d, acc, (double)p0 + (double)t0, inv);
    }
    return;
  }

  // large m: a block folds one (entry, dim slice) at a time; its row groups
  // take strided subsets of the group's tokens and are summed through LDS
  const int DS = a.ds;                 // dims of a slice (divides d, multiple of 8)
  const int nsl = a.d / DS;
  const int TS = DS >> 3;              // threads across the slice
  const int RS = kCompressThreads / TS;
  const int ls = threadIdx.x % TS;
  const int gs = threadIdx.x / TS;
  __shared__ float w_s[256];
  __shared__ float red_s[kCompressThreads];
  extern __shared__ float acc_s[];     // [RS][DS]
  const uint16_t* xs = a.x + (int64_t)b * a.xs + ls * 8;
  for (int u = blockIdx.x; u < N * nsl; u += gridDim.x) {
    const int j = u / nsl;
    const int base = (u % nsl) * DS;
    const int t0 = j * m;
    const int r = min(m, n - t0);
    // softmax weights of the group's r slots
    float a_i = -INFINITY;
    if (threadIdx.x < r) a_i = zb[t0 + threadIdx.x] + a.beta[threadIdx.x];
    red_s[threadIdx.x] = a_i;
    __syncthreads();
    for (int o = kCompressThreads / 2; o > 0; o >>= 1) {
      if (threadIdx.x < o) red_s[threadIdx.x] = fmaxf(red_s[threadIdx.x], red_s[threadIdx.x + o]);
      __syncthreads();
    }
    const float mx = red_s[0];
    __syncthreads();
    const float e = threadIdx.x < r ? expf(a_i - mx) : 0.0f;
    red_s[threadIdx.x] = e;
    w_s[threadIdx.x] = e;
    __syncthreads();
    for (int o = kCompressThreads / 2; o > 0; o >>= 1) {
      if (threadIdx.x < o) red_s[threadIdx.x] += red_s[threadIdx.x + o];
      __syncthreads();
    }
    const float tot = red_s[0];
    if (gs < RS) {
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 4
      for (int i = gs; i < r; i += RS) {
        float v[8];
        load_bf16x8(xs + (int64_t)(t0 + i) * a.d + base, v);
        const float wi = w_s[i];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = fmaf(wi, v[c], acc[c]);
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) acc_s[gs * DS + ls * 8 + c] = acc[c];
    }
    __syncthreads();
    // one thread per dim pair of the slice: sum the row groups, normalise, rotate
    const float inv_tot = 1.0f / tot;
    const double pos = (double)p0 + (double)t0;
    for (int t = threadIdx.x; t < DS / 2; t += kCompressThreads) {
      float e0 = 0.0f, e1 = 0.0f;
      for (int g = 0; g < RS; ++g) {
        e0 += acc_s[g * DS + 2 * t];
        e1 += acc_s[g * DS + 2 * t + 1];
      }
      e0 *= inv_tot;
      e1 *= inv_tot;
      float c, sn;
      rope_cs(pos, rope_inv_freq(base / 2 + t, a.d, a.theta), c, sn);
      float* o = a.out + (int64_t)b * a.os + (int64_t)j * a.d + base + 2 * t;
      o[0] = e0 * c - e1 * sn;
      o[1] = e0 * sn + e1 * c;
    }
    __syncthreads();
  }
}

hipError_t launch_compress(CompressArgs a, hipStream_t s) {
  const int n_max = (a.max_ntok + a.m - 1) / a.m;
  if (a.B == 0 || n_max == 0) return hipSuccess;
  int gx;
  size_t shm = 0;
  a.ds = a.d;
  if (a.m <= kSmallM) {
    const int RP = kCompressThreads / (a.d / 8);
    gx = (n_max + RP - 1) / RP;
    gx = gx > 2048 ? 2048 : gx;
  } else {
    // few entries (a decode step's open group): cut the dims into 64-wide slices
    if ((int64_t)n_max * a.B < 512 && a.d % 64 == 0) a.ds = 64;
    const int64_t units = (int64_t)n_max * (a.d / a.ds);
    gx = units > 4096 ? 4096 : (int)units;
    shm = (size_t)(kCompressThreads / (a.ds / 8)) * a.ds * sizeof(float);
  }
  hipLaunchKernelGGL(compress_kernel, dim3(gx, a.B), dim3(kCompressThreads), shm, s, a);
  return hipGetLastError();
}

}  // namespace hca
