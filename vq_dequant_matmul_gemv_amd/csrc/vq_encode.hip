// vq_encode.hip -- the VQ fit of one weight tensor on the GPU: group max-abs
// scales, k-means++ seeding on a subsample, Lloyd iterations, fp16 codebook,
// packed codes and the relative reconstruction error.
//
// What is computed (paper "Data-Free Vector Quantization Beats Affine
// Quantization at Matched Bytes Below 5 Bits", §2.2 The fit: d-dimensional
// subvectors, each group scaled by its maximum absolute value, a K-entry
// codebook fit by k-means with k-means++ initialization on a random subsample
// and plain Lloyd iterations; §2.3: codes packed to their true bit width;
// §2.6: relative reconstruction error as the corruption check).  The
// arithmetic is fixed so that the result does not depend on thread order:
//   * squared distances: fp32, coordinates summed in order, each subtract,
//     multiply and add rounded on its own (no fused multiply-add); ties go
//     to the lowest centroid;
//   * k-means++ draws and Lloyd means: weights and coordinates as integers in
//     units of 2^-32 (int64), whose sums are exact in any order -- a block
//     scan for the draws, atomic adds for the means -- then one fp64
//     division;
// so codes, codebook and scales are the same bits on every run.
//
// Design for gfx950: the scale pass, the assignment and the Lloyd sums are
// grid-wide and memory- or ALU-bound (the assignment costs (3d + 2) VALU
// operations per (subvector, centroid), centroids read from LDS as
// broadcasts); the k-means++ seeding is sequential over K and runs as one
// 1024-thread workgroup, each thread owning a contiguous run of the sample.

#include "vq_device.h"
#include "vq_kernels.h"

#include <algorithm>

namespace vqmi {

namespace {

constexpr double kFixedOne = 4294967296.0;  // 2^32: unit of the exact sums
constexpr int kAssignThreads = 256;
constexpr int kAssignTileBytes = 32 * 1024;  // centroids staged per LDS tile

// Squared distance in fp32, coordinates in order, no contraction into FMAs.
template <int D>
__device__ __forceinline__ float sqdist(const float* x, const float* c) {
#pragma clang fp contract(off)
  float acc = 0.f;
#pragma unroll
  for (int t = 0; t < D; ++t) {
    const float diff = x[t] - c[t];
    acc = acc + diff * diff;
  }
  return acc;
}

__device__ __forceinline__ int64_t to_fixed(float v) { return __double2ll_rn((double)v * kFixedOne); }

// D floats at byte voff + soff of a buffer (soff wave-uniform): one address
// register per lane whatever the point, so many loads can be in flight.  (The
// loaded words are reinterpreted as a whole float vector: bit-casting single
// elements of the loaded vector lost all but the first element in this
// compiler.)
template <int D>
__device__ __forceinline__ void load_point(float* x, rsrc_t r, uint32_t voff, uint32_t soff) {
  typedef float float2_v __attribute__((ext_vector_type(2)));
  if constexpr (D == 2) {
    const float2_v f = __builtin_bit_cast(float2_v, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
    x[0] = f.x;
    x[1] = f.y;
  } else {
#pragma unroll
    for (int q = 0; q < D / 4; ++q) {
      const float4_t f = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16u * q, soff, 0));
      x[4 * q] = f.x;
      x[4 * q + 1] = f.y;
      x[4 * q + 2] = f.z;
      x[4 * q + 3] = f.w;
    }
  }
}

// ---- 1. scales and subvectors: one wave per (row, group) -------------------
__global__ __launch_bounds__(256) void enc_scale_kernel(const float* __restrict__ w, int64_t n_groups, int group,
                                                        uint16_t* __restrict__ scales, float* __restrict__ pts) {
  const int lane = threadIdx.x & 63;
  const int64_t gi = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gi >= n_groups) return;
  const float* src = w + gi * group;  // groups of a row are consecutive, rows are consecutive
  float v[2];
  float m = 0.f;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = lane + 64 * k;
    v[k] = c < group ? src[c] : 0.f;
    m = fmaxf(m, fabsf(v[k]));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  const _Float16 s16 = (_Float16)m;  // round to nearest even
  const float s = (float)s16;
  if (lane == 0) scales[gi] = __builtin_bit_cast(uint16_t, s16);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = lane + 64 * k;
    if (c < group) pts[gi * group + c] = s == 0.f ? 0.f : v[k] / s;  // IEEE division
  }
}

// ---- 2. the subsample -------------------------------------------------------
// Sample point i goes to slot i, or, when `per` > 0 (the register seeding
// kernel, thread t owning points t*per ... t*per + per - 1), to slot
// (i % per) * 1024 + i / per, so that the threads' k-th points are adjacent.
__host__ __device__ inline int64_t sample_slot(int64_t i, int per) {
  return per > 0 ? (i % per) * 1024 + i / per : i;
}

template <int D>
__global__ __launch_bounds__(256) void enc_gather_kernel(const float* __restrict__ pts, int64_t n_pts,
                                                         const int32_t* __restrict__ idx, int n_s, int per,
                                                         float* __restrict__ sample) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_s) return;
  int64_t j = idx[i] % n_pts;  // indices outside [0, n) are reduced modulo n
  if (j < 0) j += n_pts;
  const int64_t slot = sample_slot(i, per);
#pragma unroll
  for (int t = 0; t < D; ++t) sample[slot * D + t] = pts[j * D + t];
}

// Inclusive scan of an int64 over the block (1024 threads, 16 waves).
__device__ __forceinline__ int64_t block_scan_i64(int64_t v, int64_t* part, int64_t& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  if (lane == 63) part[wid] = v;
  __syncthreads();
  if (wid == 0) {
    int64_t p = lane < nw ? part[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int64_t o = __shfl_up(p, off, 64);
      if (lane >= off) p += o;
    }
    if (lane < nw) part[16 + lane] = p;  // inclusive over waves
  }
  __syncthreads();
  total = part[16 + nw - 1];
  const int64_t before = wid > 0 ? part[16 + wid - 1] : 0;
  __syncthreads();  // part is reused by the next scan
  return before + v;
}

// ---- 3. k-means++ seeding: one workgroup -----------------------------------
template <int D>
__global__ __launch_bounds__(1024) void enc_kmeanspp_kernel(const float* __restrict__ sample, int n, int K,
                                                            const double* __restrict__ u, float* __restrict__ cent,
                                                            float* __restrict__ d2) {
  __shared__ int64_t part[32];
  __shared__ int chosen;
  __shared__ float cs[D];
  const int tid = threadIdx.x, nt = blockDim.x;
  const int per = (n + nt - 1) / nt;
  const int i0 = min(n, tid * per), i1 = min(n, i0 + per);
  auto draw_uniform = [&](double uj) {  // floor(u * n), kept inside the sample
    const int64_t k = (int64_t)floor(uj * (double)n);
    return (int)min<int64_t>(max<int64_t>(k, 0), n - 1);
  };
  for (int j = 0; j < K; ++j) {
    if (j == 0) {
      if (tid == 0) chosen = draw_uniform(u[0]);
    } else {
      int64_t local = 0;
      for (int i = i0; i < i1; ++i) local += to_fixed(d2[i]);
      int64_t total;
      const int64_t incl = block_scan_i64(local, part, total);
      if (total == 0) {
        if (tid == 0) chosen = draw_uniform(u[j]);
      } else {
        int64_t target = (int64_t)floor(u[j] * (double)total);
        target = min<int64_t>(max<int64_t>(target, 0), total - 1);
        const int64_t excl = incl - local;
        if (excl <= target && target < incl) {  // exactly one thread holds the target
          int64_t run = excl;
          int pick = i1 - 1;
          for (int i = i0; i < i1; ++i) {
            run += to_fixed(d2[i]);
            if (run > target) { pick = i; break; }
          }
          chosen = pick;
        }
      }
    }
    __syncthreads();
    if (tid < D) {
      cs[tid] = sample[(int64_t)chosen * D + tid];
      cent[(int64_t)j * D + tid] = cs[tid];
    }
    __syncthreads();
    float c[D];
#pragma unroll
    for (int t = 0; t < D; ++t) c[t] = cs[t];
    for (int i = i0; i < i1; ++i) {
      float x[D];
#pragma unroll
      for (int t = 0; t < D; ++t) x[t] = sample[(int64_t)i * D + t];
      const float dist = sqdist<D>(x, c);
      d2[i] = j == 0 ? dist : fminf(d2[i], dist);
    }
    __syncthreads();
  }
}

// The same seeding with each thread's squared distances in registers: up to
// P sample points per thread (n <= NT * P; the sample stored transposed, so
// the threads' k-th points are adjacent), and for d = 2 the points
// themselves in registers too, so that a step makes no global load: the
// thread owning the drawn point hands its coordinates over through LDS.  The
// draw and the arithmetic are the kernel's above, step for step.
template <int D, int P, int NT>
__global__ __launch_bounds__(NT) void enc_kmeanspp_reg_kernel(const float* __restrict__ sample, int n, int K,
                                                              const double* __restrict__ u,
                                                              float* __restrict__ cent) {
  constexpr bool XREG = D == 2;
  __shared__ int64_t part[32];
  __shared__ int chosen;
  __shared__ int from_regs;
  __shared__ float cs[D];
  const int tid = threadIdx.x;
  const int per = (n + NT - 1) / NT;
  const int i0 = min(n, tid * per), cnt = min(n, i0 + per) - i0;
  auto draw_uniform = [&](double uj) {
    const int64_t k = (int64_t)floor(uj * (double)n);
    return (int)min<int64_t>(max<int64_t>(k, 0), n - 1);
  };
  const rsrc_t rs = make_rsrc(sample, (uint64_t)NT * P * D * 4);
  const uint32_t voff = (uint32_t)tid * D * 4u;  // this thread's k-th point: slot k * NT + tid
  auto point = [&](int k, float* x) {
    if (k < cnt) load_point<D>(x, rs, voff, (uint32_t)k * NT * D * 4u);
    else
#pragma unroll
      for (int t = 0; t < D; ++t) x[t] = 0.f;
  };
  float d2[P];
  float xr[XREG ? P : 1][D];
#pragma unroll
  for (int k = 0; k < P; ++k) {
    d2[k] = 0.f;
    if constexpr (XREG) point(k, xr[k]);
  }
  for (int j = 0; j < K; ++j) {
    if (tid == 0) from_regs = 0;
    if (j == 0) {
      if (tid == 0) chosen = draw_uniform(u[j]);
    } else {
      int64_t local = 0;
#pragma unroll
      for (int k = 0; k < P; ++k)
        if (k < cnt) local += to_fixed(d2[k]);
      int64_t total;
      const int64_t incl = block_scan_i64(local, part, total);
      // the search recomputes the fixed-point weights: without this the
      // compiler keeps every point's int64 weight alive across the scan
#pragma unroll
      for (int k = 0; k < P; ++k) asm volatile("" : "+v"(d2[k]));
      if (total == 0) {
        if (tid == 0) chosen = draw_uniform(u[j]);
      } else {
        int64_t target = (int64_t)floor(u[j] * (double)total);
        target = min<int64_t>(max<int64_t>(target, 0), total - 1);
        const int64_t excl = incl - local;
        if (excl <= target && target < incl) {
          int64_t run = excl;
          bool found = false;
#pragma unroll
          for (int k = 0; k < P; ++k) {
            if (k < cnt && !found) {
              run += to_fixed(d2[k]);
              if (run > target) {
                found = true;
                chosen = i0 + k;
                if constexpr (XREG) {
#pragma unroll
                  for (int t = 0; t < D; ++t) cs[t] = xr[k][t];
                  from_regs = 1;
                }
              }
            }
          }
        }
      }
    }
    __syncthreads();
    if (tid < D && !from_regs) cs[tid] = sample[sample_slot(chosen, per) * D + tid];
    __syncthreads();
    float c[D];
#pragma unroll
    for (int t = 0; t < D; ++t) c[t] = cs[t];
    if (tid < D) cent[(int64_t)j * D + tid] = cs[tid];
    if constexpr (XREG) {
#pragma unroll
      for (int k = 0; k < P; ++k) {
        if (k < cnt) {
          const float dist = sqdist<D>(xr[k], c);
          d2[k] = j == 0 ? dist : fminf(d2[k], dist);
        }
      }
    } else {
      // batches of 32 / D points: their loads in flight together, the
      // scheduling barrier keeps the compiler from hoisting every batch's
      // loads at once
      constexpr int BP = 32 / D;
#pragma unroll
      for (int kb = 0; kb < P; kb += BP) {
        float x[BP][D];
#pragma unroll
        for (int k = 0; k < BP; ++k) point(kb + k, x[k]);
#pragma unroll
        for (int k = 0; k < BP; ++k) {
          if (kb + k < cnt) {
            const float dist = sqdist<D>(x[k], c);
            d2[kb + k] = j == 0 ? dist : fminf(d2[kb + k], dist);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
  }
}

// The seeding for d = 4 and 8 (whose points do not fit in registers beside
// everything else): squared distances in registers, the thread's points
// loaded from the transposed sample every step, in batches.
template <int D, int P, int NT>
__global__ __launch_bounds__(NT) void enc_kmeanspp_regd_kernel(const float* __restrict__ sample, int n, int K,
                                                               const double* __restrict__ u,
                                                               float* __restrict__ cent) {
  __shared__ int64_t part[32];
  __shared__ int chosen;
  __shared__ float cs[D];
  const int tid = threadIdx.x;
  const int per = (n + NT - 1) / NT;
  const int i0 = min(n, tid * per), cnt = min(n, i0 + per) - i0;
  auto draw_uniform = [&](double uj) {
    const int64_t k = (int64_t)floor(uj * (double)n);
    return (int)min<int64_t>(max<int64_t>(k, 0), n - 1);
  };
  const rsrc_t rs = make_rsrc(sample, (uint64_t)NT * P * D * 4);
  const uint32_t voff = (uint32_t)tid * D * 4u;  // this thread's k-th point: slot k * NT + tid
  float d2[P];
#pragma unroll
  for (int k = 0; k < P; ++k) d2[k] = 0.f;
  for (int j = 0; j < K; ++j) {
    if (j == 0) {
      if (tid == 0) chosen = draw_uniform(u[0]);
    } else {
      int64_t local = 0;
#pragma unroll
      for (int k = 0; k < P; ++k)
        if (k < cnt) local += to_fixed(d2[k]);
      int64_t total;
      const int64_t incl = block_scan_i64(local, part, total);
#pragma unroll
      for (int k = 0; k < P; ++k) asm volatile("" : "+v"(d2[k]));
      if (total == 0) {
        if (tid == 0) chosen = draw_uniform(u[j]);
      } else {
        int64_t target = (int64_t)floor(u[j] * (double)total);
        target = min<int64_t>(max<int64_t>(target, 0), total - 1);
        const int64_t excl = incl - local;
        if (excl <= target && target < incl) {
          int64_t run = excl;
          int pick = i0 + cnt - 1;
          bool found = false;
#pragma unroll
          for (int k = 0; k < P; ++k) {
            if (k < cnt && !found) {
              run += to_fixed(d2[k]);
              if (run > target) {
                pick = i0 + k;
                found = true;
              }
            }
          }
          chosen = pick;
        }
      }
    }
    __syncthreads();
    if (tid < D) {
      cs[tid] = sample[sample_slot(chosen, per) * D + tid];
      cent[(int64_t)j * D + tid] = cs[tid];
    }
    __syncthreads();
    float c[D];
#pragma unroll
    for (int t = 0; t < D; ++t) c[t] = cs[t];
    constexpr int BP = 32 / D;
#pragma unroll
    for (int kb = 0; kb < P; kb += BP) {
      float x[BP][D];
#pragma unroll
      for (int k = 0; k < BP; ++k) {
        if (kb + k < cnt) load_point<D>(x[k], rs, voff, (uint32_t)(kb + k) * NT * D * 4u);
        else
#pragma unroll
          for (int t = 0; t < D; ++t) x[k][t] = 0.f;
      }
#pragma unroll
      for (int k = 0; k < BP; ++k) {
        if (kb + k < cnt) {
          const float dist = sqdist<D>(x[k], c);
          d2[kb + k] = j == 0 ? dist : fminf(d2[kb + k], dist);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
  }
}

// ---- 4. assignment: nearest centroid of every subvector --------------------
template <int D>
__global__ __launch_bounds__(kAssignThreads) void enc_assign_kernel(const float* __restrict__ pts, int64_t n,
                                                                    const float* __restrict__ cent, int K,
                                                                    int32_t* __restrict__ codes) {
  constexpr int TILE = kAssignTileBytes / (4 * D);
  __shared__ __align__(16) float tile[TILE * D];
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  float x[D];
#pragma unroll
  for (int t = 0; t < D; ++t) x[t] = i < n ? pts[i * D + t] : 0.f;
  float best = __builtin_inff();
  int code = 0;
  for (int k0 = 0; k0 < K; k0 += TILE) {
    const int nk = min(TILE, K - k0);
    __syncthreads();
    for (int q = threadIdx.x; q < nk * D; q += blockDim.x) tile[q] = cent[(int64_t)k0 * D + q];
    __syncthreads();
    for (int k = 0; k < nk; ++k) {
      const float dist = sqdist<D>(x, tile + k * D);
      if (dist < best) {  // strict: ties keep the lowest index
        best = dist;
        code = k0 + k;
      }
    }
  }
  if (i < n) codes[i] = code;
}

// ---- 5. Lloyd sums (exact) and the new centroids ---------------------------
// LDS holds the block's sums when K * (D + 1) * 8 bytes fit in kAccumLds.
constexpr int kAccumLds = 48 * 1024;

template <int D, bool kLds>
__global__ __launch_bounds__(256) void enc_accum_kernel(const float* __restrict__ pts, const int32_t* __restrict__ codes,
                                                        int64_t n, int K, unsigned long long* __restrict__ sums,
                                                        unsigned long long* __restrict__ counts) {
  __shared__ unsigned long long ls[kLds ? kAccumLds / 8 : 1];
  unsigned long long* s = kLds ? ls : sums;
  unsigned long long* c = kLds ? ls + (int64_t)K * D : counts;
  if constexpr (kLds) {
    for (int q = threadIdx.x; q < K * (D + 1); q += blockDim.x) ls[q] = 0ull;
    __syncthreads();
  }
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int k = codes[i];
#pragma unroll
    for (int t = 0; t < D; ++t) atomicAdd(s + (int64_t)k * D + t, (unsigned long long)to_fixed(pts[i * D + t]));
    atomicAdd(c + k, 1ull);
  }
  if constexpr (kLds) {
    __syncthreads();
    for (int q = threadIdx.x; q < K * (D + 1); q += blockDim.x) {
      const unsigned long long v = ls[q];
      if (v == 0ull) continue;
      if (q < K * D) atomicAdd(sums + q, v);
      else atomicAdd(counts + (q - K * D), v);
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void enc_mean_kernel(const unsigned long long* __restrict__ sums,
                                                       const unsigned long long* __restrict__ counts, int K,
                                                       float* __restrict__ cent) {
  const int q = blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= K * D) return;
  const int64_t n = (int64_t)counts[q / D];
  if (n == 0) return;  // an empty cluster keeps its centroid
  const double s = (double)(int64_t)sums[q];
  cent[q] = (float)(s / (double)n / kFixedOne);
}

// ---- 6. fp16 codebook (and its fp32 values for the final assignment) -------
__global__ __launch_bounds__(256) void enc_codebook_kernel(float* __restrict__ cent, uint16_t* __restrict__ cb,
                                                           int n) {
  const int q = blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= n) return;
  const _Float16 h = (_Float16)cent[q];
  cb[q] = __builtin_bit_cast(uint16_t, h);
  cent[q] = (float)h;
}

// ---- 7. packing: one thread per 32-code block of B words -------------------
__global__ __launch_bounds__(256) void enc_pack_kernel(const int32_t* __restrict__ codes, int64_t n_blocks, int B,
                                                       uint32_t* __restrict__ words) {
  const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= n_blocks) return;
  uint32_t out[16];
  for (int q = 0; q < B; ++q) out[q] = 0u;
  for (int j = 0; j < 32; ++j) {
    const uint32_t v = (uint32_t)codes[blk * 32 + j];
    const int bit = j * B, wi = bit >> 5, sh = bit & 31;
    out[wi] |= v << sh;
    if (sh + B > 32) out[wi + 1] |= v >> (32 - sh);
  }
  for (int q = 0; q < B; ++q) words[blk * B + q] = out[q];
}

// ---- 8. relative reconstruction error --------------------------------------
template <int D>
__global__ __launch_bounds__(256) void enc_relerr_kernel(const float* __restrict__ w, const int32_t* __restrict__ codes,
                                                         const uint16_t* __restrict__ cb,
                                                         const uint16_t* __restrict__ scales, int64_t n_pts,
                                                         int pts_per_group, double* __restrict__ acc) {
  double num = 0.0, den = 0.0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_pts; i += (int64_t)gridDim.x * blockDim.x) {
    const float s = half_bits_to_float(scales[i / pts_per_group]);
    const int k = codes[i];
#pragma unroll
    for (int t = 0; t < D; ++t) {
      const _Float16 wq = (_Float16)(half_bits_to_float(cb[k * D + t]) * s);  // the dequantized weight
      const double a = (double)w[i * D + t], e = a - (double)(float)wq;
      num += e * e;
      den += a * a;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    num += __shfl_xor(num, off, 64);
    den += __shfl_xor(den, off, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    atomicAdd(acc, num);
    atomicAdd(acc + 1, den);
  }
}

__global__ void enc_relerr_final_kernel(const double* __restrict__ acc, double* __restrict__ out) {
  *out = acc[1] > 0.0 ? sqrt(acc[0] / acc[1]) : 0.0;
}

int num_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
  }
  return n;
}

// Workspace segments, each 256-byte aligned.
struct EncWs {
  float* pts;
  int32_t* codes;
  float* sample;
  float* d2;
  float* cent;
  unsigned long long* sums;    // [K][D] then counts [K]
  double* acc;                 // 2 relerr sums
  size_t bytes;
};

EncWs enc_layout(void* base, int64_t n_pts, int d, int K, int n_s) {
  EncWs ws{};
  size_t off = 0;
  auto take = [&](size_t b) {
    const size_t o = off;
    off += (b + 255) & ~(size_t)255;
    return static_cast<uint8_t*>(base) + o;
  };
  ws.pts = reinterpret_cast<float*>(take((size_t)n_pts * d * 4));
  ws.codes = reinterpret_cast<int32_t*>(take((size_t)n_pts * 4));
  ws.sample = reinterpret_cast<float*>(take((size_t)n_s * d * 4));
  ws.d2 = reinterpret_cast<float*>(take((size_t)n_s * 4));
  ws.cent = reinterpret_cast<float*>(take((size_t)K * d * 4));
  ws.sums = reinterpret_cast<unsigned long long*>(take((size_t)K * (d + 1) * 8));
  ws.acc = reinterpret_cast<double*>(take(16));
  ws.bytes = off;
  return ws;
}

#define VQMI_CHECK(e)                    \
  do {                                   \
    hipError_t err_ = (e);               \
    if (err_ != hipSuccess) return err_; \
  } while (0)

template <int D>
hipError_t encode_d(const float* w, int rows, int cols, int log2_k, int group, const int32_t* sample_idx, int n_s,
                    const double* uniforms, int iters, uint32_t* codes_out, uint16_t* cb_out, uint16_t* scales_out,
                    double* relerr, void* workspace, hipStream_t s) {
  const int K = 1 << log2_k;
  const int64_t n_pts = (int64_t)rows * cols / D;
  const EncWs ws = enc_layout(workspace, n_pts, D, K, n_s);
  unsigned long long* counts = ws.sums + (int64_t)K * D;
  const int64_t n_groups = (int64_t)rows * cols / group;
  hipLaunchKernelGGL(enc_scale_kernel, dim3((unsigned)((n_groups + 3) / 4)), dim3(256), 0, s, w, n_groups, group,
                     scales_out, ws.pts);
  VQMI_CHECK(hipGetLastError());
  const bool reg_seeding = n_s <= 1024 * 16;  // the register seeding kernel reads the sample transposed
  hipLaunchKernelGGL(enc_gather_kernel<D>, dim3((n_s + 255) / 256), dim3(256), 0, s, ws.pts, n_pts, sample_idx, n_s,
                     reg_seeding ? (n_s + 1023) / 1024 : 0, ws.sample);
  VQMI_CHECK(hipGetLastError());
  // seeding: squared distances in registers for up to 16,384 sample points
  // (16 per thread), in the workspace beyond that
  if (reg_seeding) {
    if constexpr (D == 2)
      hipLaunchKernelGGL((enc_kmeanspp_reg_kernel<D, 16, 1024>), dim3(1), dim3(1024), 0, s, ws.sample, n_s, K,
                         uniforms, ws.cent);
    else
      hipLaunchKernelGGL((enc_kmeanspp_regd_kernel<D, 16, 1024>), dim3(1), dim3(1024), 0, s, ws.sample, n_s, K,
                         uniforms, ws.cent);
  } else
    hipLaunchKernelGGL(enc_kmeanspp_kernel<D>, dim3(1), dim3(1024), 0, s, ws.sample, n_s, K, uniforms, ws.cent, ws.d2);
  VQMI_CHECK(hipGetLastError());
  const unsigned assign_blocks = (unsigned)((n_pts + kAssignThreads - 1) / kAssignThreads);
  const bool lds = (int64_t)K * (D + 1) * 8 <= kAccumLds;
  const unsigned accum_blocks = (unsigned)std::min<int64_t>((n_pts + 255) / 256, (int64_t)num_cus() * (lds ? 2 : 8));
  for (int it = 0; it < iters; ++it) {
    hipLaunchKernelGGL(enc_assign_kernel<D>, dim3(assign_blocks), dim3(kAssignThreads), 0, s, ws.pts, n_pts, ws.cent,
                       K, ws.codes);
    VQMI_CHECK(hipGetLastError());
    VQMI_CHECK(launch_zero(ws.sums, (size_t)K * (D + 1) * 8, s));
    if (lds)
      hipLaunchKernelGGL((enc_accum_kernel<D, true>), dim3(accum_blocks), dim3(256), 0, s, ws.pts, ws.codes, n_pts, K,
                         ws.sums, counts);
    else
      hipLaunchKernelGGL((enc_accum_kernel<D, false>), dim3(accum_blocks), dim3(256), 0, s, ws.pts, ws.codes, n_pts,
                         K, ws.sums, counts);
    VQMI_CHECK(hipGetLastError());
    hipLaunchKernelGGL(enc_mean_kernel<D>, dim3((K * D + 255) / 256), dim3(256), 0, s, ws.sums, counts, K, ws.cent);
    VQMI_CHECK(hipGetLastError());
  }
  hipLaunchKernelGGL(enc_codebook_kernel, dim3((K * D + 255) / 256), dim3(256), 0, s, ws.cent, cb_out, K * D);
  VQMI_CHECK(hipGetLastError());
  hipLaunchKernelGGL(enc_assign_kernel<D>, dim3(assign_blocks), dim3(kAssignThreads), 0, s, ws.pts, n_pts, ws.cent, K,
                     ws.codes);
  VQMI_CHECK(hipGetLastError());
  const int64_t n_blocks = n_pts / 32;
  hipLaunchKernelGGL(enc_pack_kernel, dim3((unsigned)((n_blocks + 255) / 256)), dim3(256), 0, s, ws.codes, n_blocks,
                     log2_k, codes_out);
  VQMI_CHECK(hipGetLastError());
  VQMI_CHECK(launch_zero(ws.acc, 16, s));
  const unsigned rel_blocks = (unsigned)std::min<int64_t>((n_pts + 255) / 256, (int64_t)num_cus() * 4);
  hipLaunchKernelGGL(enc_relerr_kernel<D>, dim3(rel_blocks), dim3(256), 0, s, w, ws.codes, cb_out, scales_out, n_pts,
                     group / D, ws.acc);
  VQMI_CHECK(hipGetLastError());
  hipLaunchKernelGGL(enc_relerr_final_kernel, dim3(1), dim3(1), 0, s, ws.acc, relerr);
  return hipGetLastError();
}

}  // namespace

size_t encode_workspace_bytes(int rows, int cols, int d, int log2_k, int n_sample) {
  return enc_layout(nullptr, (int64_t)rows * cols / d, d, 1 << log2_k, n_sample).bytes;
}

hipError_t launch_encode(const float* w, int rows, int cols, int d, int log2_k, int group, const int32_t* sample_idx,
                         int n_sample, const double* uniforms, int iters, uint32_t* codes, uint16_t* codebook,
                         uint16_t* scales, double* relerr, void* workspace, hipStream_t s) {
  switch (d) {
    case 2: return encode_d<2>(w, rows, cols, log2_k, group, sample_idx, n_sample, uniforms, iters, codes, codebook,
                               scales, relerr, workspace, s);
    case 4: return encode_d<4>(w, rows, cols, log2_k, group, sample_idx, n_sample, uniforms, iters, codes, codebook,
                               scales, relerr, workspace, s);
    case 8: return encode_d<8>(w, rows, cols, log2_k, group, sample_idx, n_sample, uniforms, iters, codes, codebook,
                               scales, relerr, workspace, s);
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace vqmi
