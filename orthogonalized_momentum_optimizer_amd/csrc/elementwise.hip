// HBM-bound kernels of the Muon step: the fused momentum kernel, the per-matrix norm
// finish and the parameter update.
//
// Momentum and Nesterov follow the optimizer of page
// "深入解析KellerJordan/modded-nanogpt中的训练架构与优化技术" (section
// "Muon优化器：动量正交化技术", subsection "核心算法": standard SGD momentum, nesterov on by
// default); the Frobenius pre-normalisation is the reading recorded in muon.h.
//
// Layout: every kernel works on 64x64 tiles, 256 threads, each thread owning four
// consecutive columns of four rows (rows t/16 + 16k, columns 4*(t%16)..+3), so a wavefront
// reads 256 contiguous bytes of fp32 per row segment; the update of matrices whose column
// count is a multiple of 8 uses eight columns of two rows per thread instead (16-byte bf16
// accesses, measured 10% faster). Tall matrices are transposed through an LDS tile so that
// both the original-orientation side and the wide-form side of the copy stay coalesced.
#include "muon_internal.h"

namespace muon {
namespace {

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> two bfloat16 in one dword (lo = first), round to nearest even, NaN stays
// NaN: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Element index of (r, c) in the workspace matrix X (np columns): the tiled layout for
// bf16, row-major for fp32. Four consecutive columns from a multiple of 4 stay contiguous.
template <int XDT>
__device__ __forceinline__ size_t xidx(int r, int c, int np) {
  return XDT == 0 ? toff(r, c, np) : (size_t)r * np + c;
}

template <int DT>
__device__ __forceinline__ float load1(const void* p, size_t i) {
  if (DT == 0) return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
  return static_cast<const float*>(p)[i];
}

template <int DT>
__device__ __forceinline__ void load4(const void* p, size_t i, float v[4]) {
  if (DT == 0) {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
    v[0] = bf16_bits_to_f32(w.x & 0xffffu);
    v[1] = bf16_bits_to_f32(w.x >> 16);
    v[2] = bf16_bits_to_f32(w.y & 0xffffu);
    v[3] = bf16_bits_to_f32(w.y >> 16);
  } else {
    const float4 w = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
  }
}

template <int DT>
__device__ __forceinline__ void store1(void* p, size_t i, float v) {
  if (DT == 0) static_cast<uint16_t*>(p)[i] = (uint16_t)(pack_bf16(v, 0.f) & 0xffffu);
  else static_cast<float*>(p)[i] = v;
}

template <int DT>
__device__ __forceinline__ void store4(void* p, size_t i, const float v[4]) {
  if (DT == 0) {
    uint2 w;
    w.x = pack_bf16(v[0], v[1]);
    w.y = pack_bf16(v[2], v[3]);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + i) = w;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(p) + i) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Sum of the squares of four fp32 values in double: each square is exact in double (24-bit
// significands give at most 48 bits), so the per-tile sums neither overflow nor underflow
// for any finite fp32 input, and the order of the additions is fixed.
__device__ __forceinline__ double sumsq4(const float v[4]) {
  const double a = v[0], b = v[1], c = v[2], d = v[3];
  return (a * a + b * b) + (c * c + d * d);
}

// One 64x64 tile of the padded wide form X (mp x np) per block, matrix q = blockIdx.y.
// Momentum (in place), U, the tile's sum of U^2 (in double), and X0 = U stored in the wide
// form; padding positions of X0 receive zeros. GDT: grad dtype, XDT: X dtype (0 bf16, 1 f32).
template <int GDT, int XDT>
__global__ __launch_bounds__(256) void momentum_kernel(ElemLaunch L) {
  __shared__ float tile[kTile][kTile + 1];
  __shared__ double red[4];
  const int q = blockIdx.y;
  const int t = threadIdx.x;
  const int tiles_n = L.np / kTile;
  const int ti = blockIdx.x / tiles_n, tj = blockIdx.x % tiles_n;  // wide tile coordinates
  const int r0 = L.tall ? tj * kTile : ti * kTile;                  // original-orientation origin
  const int c0 = L.tall ? ti * kTile : tj * kTile;
  const void* g = L.in[q];
  float* mom = L.mom[q];
  void* x = static_cast<char*>(L.x) + (size_t)q * L.mp * L.np * (XDT == 0 ? 2 : 4);
  const float beta = L.beta;
  const int lc = 4 * (t & 15);
  double ss = 0.0;

#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int lr = (t >> 4) + 16 * k;
    const int r = r0 + lr, c = c0 + lc;
    float u[4] = {0.f, 0.f, 0.f, 0.f};
    if (r < L.rows) {
      const size_t base = (size_t)r * L.cols + c;
      if (L.vec) {
        if (c < L.cols) {
          float gv[4];
          load4<GDT>(g, base, gv);
          if (mom) {
            float4 mv = *reinterpret_cast<const float4*>(mom + base);
            float m4[4] = {mv.x, mv.y, mv.z, mv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              m4[e] = fmaf(beta, m4[e], gv[e]);
              u[e] = L.nesterov ? fmaf(beta, m4[e], gv[e]) : m4[e];
            }
            *reinterpret_cast<float4*>(mom + base) = make_float4(m4[0], m4[1], m4[2], m4[3]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) u[e] = gv[e];
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (c + e < L.cols) {
            const float gv = load1<GDT>(g, base + e);
            if (mom) {
              const float m = fmaf(beta, mom[base + e], gv);
              mom[base + e] = m;
              u[e] = L.nesterov ? fmaf(beta, m, gv) : m;
            } else {
              u[e] = gv;
            }
          }
        }
      }
    }
    if (!L.tall) {
      ss += sumsq4(u);
      store4<XDT>(x, xidx<XDT>(r, c, L.np), u);  // wide (i, j) = (r, c); r < mp, c < np
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) tile[lr][lc + e] = u[e];
    }
  }

  if (L.tall) {
    __syncthreads();
    // the sum of squares is taken over the wide form, element for element in the order of
    // the wide path, so a matrix and its transpose give bitwise the same partial sums
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int a = (t >> 4) + 16 * k;  // wide row (original column) within the tile
      const int b = 4 * (t & 15);       // wide column (original row) within the tile
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = tile[b + e][a];
      ss += sumsq4(v);
      store4<XDT>(x, xidx<XDT>(c0 + a, r0 + b, L.np), v);
    }
  }

  ss = wave_sum(ss);
  if ((t & 63) == 0) red[t >> 6] = ss;
  __syncthreads();
  if (t == 0) {
    const int tiles = (L.mp / kTile) * tiles_n;
    L.partials[(size_t)q * tiles + blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
  }
}

// One block per matrix: nu = sqrt(sum of tile partials) in double, in a fixed order, and the
// scales s1 = 1/(nu + eps), s2 = s1^2 that the first round folds into its products.
//
// X0 holds U itself (unnormalised), and the first round's Gram product accumulates the
// products of its entries in fp32: entries near fp32's range limits would overflow (|U| of
// about 1e17 and more) or underflow (squares below 2^-126) there before s2 is applied. A
// matrix whose nu lies outside [2^-40, 2^40] therefore has its X0 rescaled here by the exact
// power of two 2^-k, k = floor(log2 nu) (so its entries are below 2 in magnitude), and
// s1 = 2^k / (nu + eps): X0 s1 is the same U / (nu + eps). Inside that range nothing is
// rescaled (every Gram entry and partial product then lies between 2^-110 and 2^95, for any
// K up to 2^15); the rescale is one block's pass over the matrix, taken only for such inputs.
__global__ __launch_bounds__(256) void norm_kernel(const double* partials, int tiles,
                                                   float* scales, float eps, void* x0,
                                                   size_t mn, int x_f32) {
  __shared__ double red[4];
  __shared__ int kexp;
  const int q = blockIdx.x, t = threadIdx.x;
  const double* p = partials + (size_t)q * tiles;
  double s = 0.0;
  for (int i = t; i < tiles; i += 256) s += p[i];
  s = wave_sum(s);
  if ((t & 63) == 0) red[t >> 6] = s;
  __syncthreads();
  if (t == 0) {
    const double tot = (red[0] + red[1]) + (red[2] + red[3]);
    const double nu = sqrt(tot);
    int k = 0;
    if (nu > 0.0 && nu <= 1.7976931348623157e308 && (nu < 0x1p-40 || nu > 0x1p40))
      k = ilogb(nu);  // nu 2^-k in [1, 2); |k| >= 40 here
    const double s1 = ldexp(1.0, k) / (nu + (double)eps);
    scales[4 * q + 0] = (float)s1;
    scales[4 * q + 1] = (float)(s1 * s1);
    scales[4 * q + 2] = (float)nu;
    scales[4 * q + 3] = 0.f;
    kexp = k;
  }
  __syncthreads();
  const int k = kexp;
  if (k == 0) return;
  // X0 <- X0 2^-k, exact (the results are representable: their magnitudes are below 2)
  const double f = ldexp(1.0, -k);
  if (x_f32) {
    float4* x = reinterpret_cast<float4*>(static_cast<float*>(x0) + (size_t)q * mn);
    for (size_t i = t; i < mn / 4; i += 256) {
      float4 v = x[i];
      v.x = (float)(v.x * f); v.y = (float)(v.y * f);
      v.z = (float)(v.z * f); v.w = (float)(v.w * f);
      x[i] = v;
    }
  } else {
    uint4* x = reinterpret_cast<uint4*>(static_cast<uint16_t*>(x0) + (size_t)q * mn);
    for (size_t i = t; i < mn / 8; i += 256) {
      uint4 w = x[i];
      uint32_t* h = reinterpret_cast<uint32_t*>(&w);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = (float)(bf16_bits_to_f32(h[e] & 0xffffu) * f);
        const float hi = (float)(bf16_bits_to_f32(h[e] >> 16) * f);
        h[e] = pack_bf16(lo, hi);
      }
      x[i] = w;
    }
  }
}

// Row equaliser, pass 1: the sum of O^2 over each row of O in the caller's orientation,
// O = X (or X^T for tall matrices) [* s1]; matrix q = blockIdx.y. Each slot owns
// kRowParts x np floats of rowsum: partial sums, added in a fixed order by pass 2.
// Wide matrices: one wavefront per row of X, 16-byte loads along the row (the padding
// columns of X hold zeros, so vectors that cross cols read zeros); one partial.
// Tall matrices: a row of O is a column of X; a block owns 256 columns and one of
// kRowParts slices of X's rows (blockIdx.z); lane l of wave w sums columns 4l..4l+3 over
// rows w, w+4, ... of its slice, and the four waves' sums are added in a fixed order.
template <int XDT>
__global__ __launch_bounds__(256) void rowstat_kernel(ElemLaunch L) {
  __shared__ float part[4][256];
  const int q = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const void* x = static_cast<const char*>(L.x) + (size_t)q * L.mp * L.np * (XDT == 0 ? 2 : 4);
  float* out = L.rowsum + (size_t)q * kRowParts * L.np;
  const float s = L.apply_scale ? L.scales[4 * q] : 1.f;
  if (!L.tall) {
    const int i = blockIdx.x * 4 + w;
    if (i >= L.rows) return;
    float acc = 0.f;
    for (int c = 4 * lane; c < L.cols; c += 256) {
      float v[4];
      load4<XDT>(x, xidx<XDT>(i, c, L.np), v);
      acc += (v[0] * v[0] + v[1] * v[1]) + (v[2] * v[2] + v[3] * v[3]);
    }
    acc = wave_sum(acc);
    if (lane == 0) out[i] = acc * (s * s);
    return;
  }
  const int c0 = blockIdx.x * 256 + 4 * lane;
  const int slice = (L.cols + kRowParts - 1) / kRowParts;
  const int r_end = min(L.cols, (int)(blockIdx.z + 1) * slice);
  float a[4] = {0.f, 0.f, 0.f, 0.f};
  if (c0 < L.np) {
    for (int r = blockIdx.z * slice + w; r < r_end; r += 4) {
      float v[4];
      load4<XDT>(x, xidx<XDT>(r, c0, L.np), v);
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = fmaf(v[e], v[e], a[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) part[w][4 * lane + e] = a[e];
  __syncthreads();
  const int i = blockIdx.x * 256 + t;
  if (i < L.rows)
    out[(size_t)blockIdx.z * L.np + i] =
        ((part[0][t] + part[1][t]) + (part[2][t] + part[3][t])) * (s * s);
}

// Row equaliser, pass 2, one block per matrix q: v_i <- beta v_i + (1 - beta) rowsum_i / cols
// (the caller's state, in place), d_i = 1 / (sqrt(v_i) + eps) (0 where that is 0: such a row
// of O is zero), gamma = sqrt(sum_i rowsum_i / sum_i d_i^2 rowsum_i) in double and a fixed
// order (0 when O is zero), rowf[q * np + i] = gamma d_i.
__global__ __launch_bounds__(1024) void roweq_finish_kernel(ElemLaunch L) {
  __shared__ double red[2][16];
  const int q = blockIdx.x, t = threadIdx.x;
  const float* rs = L.rowsum + (size_t)q * kRowParts * L.np;
  const int parts = L.tall ? kRowParts : 1;
  float* f = L.rowf + (size_t)q * L.np;
  float* v = L.rowvar[q];
  const float inv_cols = 1.f / (float)L.cols;
  const float keep = 1.f - L.row_beta;
  double e = 0.0, e2 = 0.0;
  for (int i = t; i < L.rows; i += 1024) {
    float sum = rs[i];
    for (int k = 1; k < parts; ++k) sum += rs[(size_t)k * L.np + i];
    const float vi = fmaf(L.row_beta, v[i], keep * (sum * inv_cols));
    v[i] = vi;
    const float den = sqrtf(vi) + L.row_eps;
    const float di = den > 0.f ? 1.f / den : 0.f;
    f[i] = di;
    e += (double)sum;
    e2 += (double)di * (double)di * (double)sum;
  }
  e = wave_sum(e);
  e2 = wave_sum(e2);
  if ((t & 63) == 0) {
    red[0][t >> 6] = e;
    red[1][t >> 6] = e2;
  }
  __syncthreads();
  double te = 0.0, te2 = 0.0;
  for (int k = 0; k < 16; ++k) {
    te += red[0][k];
    te2 += red[1][k];
  }
  const float gamma = te2 > 0.0 ? (float)sqrt(te / te2) : 0.f;
  for (int i = t; i < L.rows; i += 1024) f[i] *= gamma;
}

// One 64x64 tile of the original orientation per block, matrix q = blockIdx.y:
// O = X (or X^T for tall matrices) [* s1] [* rowf_i], W <- W - lr * O, optional O output.
// PDT: param dtype, ODT: dtype of the O output, XDT: X dtype.
template <int PDT, int ODT, int XDT>
__global__ __launch_bounds__(256) void update_kernel(ElemLaunch L) {
  __shared__ float tile[kTile][kTile + 1];
  const int q = blockIdx.y;
  const int t = threadIdx.x;
  const int tiles_c = (L.cols + kTile - 1) / kTile;
  const int r0 = (blockIdx.x / tiles_c) * kTile, c0 = (blockIdx.x % tiles_c) * kTile;
  const void* x = static_cast<const char*>(L.x) + (size_t)q * L.mp * L.np * (XDT == 0 ? 2 : 4);
  void* w = L.param[q];
  void* o = L.out[q];
  // a failed single launch of the rounds (L.fault set) makes O, and so W, NaN
  const float s = (L.fault && *L.fault != 0u) ? __builtin_nanf("")
                  : L.apply_scale ? L.scales[4 * q] : 1.f;
  const float lr = L.lr;
  const float* rowf = L.rowf ? L.rowf + (size_t)q * L.np : nullptr;

  if (L.tall) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int a = (t >> 4) + 16 * k, b = 4 * (t & 15);
      float v[4];
      load4<XDT>(x, xidx<XDT>(c0 + a, r0 + b, L.np), v);  // within the padded buffer
#pragma unroll
      for (int e = 0; e < 4; ++e) tile[a][b + e] = v[e];
    }
    __syncthreads();
  }

  const int lc = 4 * (t & 15);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int lr_ = (t >> 4) + 16 * k;
    const int r = r0 + lr_, c = c0 + lc;
    if (r >= L.rows) continue;
    float ov[4];
    if (L.tall) {
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[e] = tile[lc + e][lr_];
    } else {
      load4<XDT>(x, xidx<XDT>(r, c, L.np), ov);
    }
    const float sr = rowf ? s * rowf[r] : s;
#pragma unroll
    for (int e = 0; e < 4; ++e) ov[e] *= sr;
    const size_t base = (size_t)r * L.cols + c;
    if (L.vec) {
      if (c >= L.cols) continue;
      if (w) {
        float wv[4];
        load4<PDT>(w, base, wv);
#pragma unroll
        for (int e = 0; e < 4; ++e) wv[e] = fmaf(-lr, ov[e], wv[e]);
        store4<PDT>(w, base, wv);
      }
      if (o) store4<ODT>(o, base, ov);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (c + e >= L.cols) break;
        if (w) store1<PDT>(w, base + e, fmaf(-lr, ov[e], load1<PDT>(w, base + e)));
        if (o) store1<ODT>(o, base + e, ov[e]);
      }
    }
  }
}

// Eight consecutive elements (16 bytes of bf16, 32 of fp32) from an index that is a
// multiple of 8.
template <int DT>
__device__ __forceinline__ void load8(const void* p, size_t i, float v[8]) {
  if (DT == 0) {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = bf16_bits_to_f32(u[k] & 0xffffu);
      v[2 * k + 1] = bf16_bits_to_f32(u[k] >> 16);
    }
  } else {
    const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    const float4 a = q[0], b = q[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <int DT>
__device__ __forceinline__ void store8(void* p, size_t i, const float v[8]) {
  if (DT == 0) {
    uint4 w;
    w.x = pack_bf16(v[0], v[1]);
    w.y = pack_bf16(v[2], v[3]);
    w.z = pack_bf16(v[4], v[5]);
    w.w = pack_bf16(v[6], v[7]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p) + i) = w;
  } else {
    float4* q = reinterpret_cast<float4*>(static_cast<float*>(p) + i);
    q[0] = make_float4(v[0], v[1], v[2], v[3]);
    q[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// The update for matrices whose cols is a multiple of 8: each thread owns eight consecutive
// columns of two rows (rows t/8 + 32k, columns 8*(t%8)..+7), 16-byte bf16 accesses.
template <int PDT, int ODT, int XDT>
__global__ __launch_bounds__(256) void update_kernel8(ElemLaunch L) {
  __shared__ float tile[kTile][kTile + 1];
  const int q = blockIdx.y;
  const int t = threadIdx.x;
  const int tiles_c = (L.cols + kTile - 1) / kTile;
  const int r0 = (blockIdx.x / tiles_c) * kTile, c0 = (blockIdx.x % tiles_c) * kTile;
  const void* x = static_cast<const char*>(L.x) + (size_t)q * L.mp * L.np * (XDT == 0 ? 2 : 4);
  void* w = L.param[q];
  void* o = L.out[q];
  // a failed single launch of the rounds (L.fault set) makes O, and so W, NaN
  const float s = (L.fault && *L.fault != 0u) ? __builtin_nanf("")
                  : L.apply_scale ? L.scales[4 * q] : 1.f;
  const float lr = L.lr;
  const float* rowf = L.rowf ? L.rowf + (size_t)q * L.np : nullptr;

  if (L.tall) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int a = (t >> 4) + 16 * k, b = 4 * (t & 15);
      float v[4];
      load4<XDT>(x, xidx<XDT>(c0 + a, r0 + b, L.np), v);  // within the padded buffer
#pragma unroll
      for (int e = 0; e < 4; ++e) tile[a][b + e] = v[e];
    }
    __syncthreads();
  }

  const int lc = 8 * (t & 7);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int lr_ = (t >> 3) + 32 * k;
    const int r = r0 + lr_, c = c0 + lc;
    if (r >= L.rows || c >= L.cols) continue;  // cols % 8 == 0: the whole vector is inside
    float ov[8];
    if (L.tall) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ov[e] = tile[lc + e][lr_];
    } else {
      load8<XDT>(x, xidx<XDT>(r, c, L.np), ov);
    }
    const float sr = rowf ? s * rowf[r] : s;
#pragma unroll
    for (int e = 0; e < 8; ++e) ov[e] *= sr;
    const size_t base = (size_t)r * L.cols + c;
    if (w) {
      float wv[8];
      load8<PDT>(w, base, wv);
#pragma unroll
      for (int e = 0; e < 8; ++e) wv[e] = fmaf(-lr, ov[e], wv[e]);
      store8<PDT>(w, base, wv);
    }
    if (o) store8<ODT>(o, base, ov);
  }
}

}  // namespace

hipError_t launch_momentum(const ElemLaunch& L, int grad_dt, int x_f32, hipStream_t s) {
  const dim3 grid((L.mp / kTile) * (L.np / kTile), L.count), block(256);
  if (grad_dt == 0 && !x_f32) launch_k((momentum_kernel<0, 0>), grid, block, 0, s, L);
  else if (grad_dt == 0) launch_k((momentum_kernel<0, 1>), grid, block, 0, s, L);
  else if (!x_f32) launch_k((momentum_kernel<1, 0>), grid, block, 0, s, L);
  else launch_k((momentum_kernel<1, 1>), grid, block, 0, s, L);
  return hipGetLastError();
}

hipError_t launch_norm(const double* partials, int tiles, float* scales, int count, float eps,
                       void* x0, size_t mn, int x_f32, hipStream_t s) {
  launch_k(norm_kernel, dim3(count), dim3(256), 0, s, partials, tiles, scales, eps, x0, mn,
           x_f32);
  return hipGetLastError();
}

hipError_t launch_rowstat(const ElemLaunch& L, int x_f32, hipStream_t s) {
  const int bx = L.tall ? (L.rows + 255) / 256 : (L.rows + 3) / 4;
  const dim3 grid(bx, L.count, L.tall ? kRowParts : 1), block(256);
  if (x_f32) launch_k(rowstat_kernel<1>, grid, block, 0, s, L);
  else launch_k(rowstat_kernel<0>, grid, block, 0, s, L);
  return hipGetLastError();
}

hipError_t launch_roweq_finish(const ElemLaunch& L, hipStream_t s) {
  launch_k(roweq_finish_kernel, dim3(L.count), dim3(1024), 0, s, L);
  return hipGetLastError();
}

hipError_t launch_update(const ElemLaunch& L, int param_dt, int out_dt, int x_f32,
                         hipStream_t s) {
  const int tiles = ((L.rows + kTile - 1) / kTile) * ((L.cols + kTile - 1) / kTile);
  const dim3 grid(tiles, L.count), block(256);
  const int code = param_dt * 4 + out_dt * 2 + x_f32;
  if (L.vec && (L.cols & 7) == 0) {
    switch (code) {
      case 0: launch_k((update_kernel8<0, 0, 0>), grid, block, 0, s, L); break;
      case 1: launch_k((update_kernel8<0, 0, 1>), grid, block, 0, s, L); break;
      case 2: launch_k((update_kernel8<0, 1, 0>), grid, block, 0, s, L); break;
      case 3: launch_k((update_kernel8<0, 1, 1>), grid, block, 0, s, L); break;
      case 4: launch_k((update_kernel8<1, 0, 0>), grid, block, 0, s, L); break;
      case 5: launch_k((update_kernel8<1, 0, 1>), grid, block, 0, s, L); break;
      case 6: launch_k((update_kernel8<1, 1, 0>), grid, block, 0, s, L); break;
      default: launch_k((update_kernel8<1, 1, 1>), grid, block, 0, s, L); break;
    }
    return hipGetLastError();
  }
  switch (code) {
    case 0: launch_k((update_kernel<0, 0, 0>), grid, block, 0, s, L); break;
    case 1: launch_k((update_kernel<0, 0, 1>), grid, block, 0, s, L); break;
    case 2: launch_k((update_kernel<0, 1, 0>), grid, block, 0, s, L); break;
    case 3: launch_k((update_kernel<0, 1, 1>), grid, block, 0, s, L); break;
    case 4: launch_k((update_kernel<1, 0, 0>), grid, block, 0, s, L); break;
    case 5: launch_k((update_kernel<1, 0, 1>), grid, block, 0, s, L); break;
    case 6: launch_k((update_kernel<1, 1, 0>), grid, block, 0, s, L); break;
    default: launch_k((update_kernel<1, 1, 1>), grid, block, 0, s, L); break;
  }
  return hipGetLastError();
}

}  // namespace muon
