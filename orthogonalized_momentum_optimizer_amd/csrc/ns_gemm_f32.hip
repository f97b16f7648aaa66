// fp32 Newton-Schulz products: the debug precision of the library.
//
// The same three products as the bf16 path (gram A = s2 X X^T, poly B = bA + cAA, apply
// X' = s1(aX + BX); page "深入解析KellerJordan/modded-nanogpt中的训练架构与优化技术",
// section "Newton-Schulz正交化"), with fp32 storage and fp32 fused multiply-adds on the
// vector ALUs. Its purpose is to separate the method from its bf16 rounding, so it favours
// plainness over speed: full 64x64 output tiles (no symmetric half), K steps of 16 through
// LDS, 256 threads each computing a 4x4 strided sub-tile. Because every product A[i][j] and
// A[j][i] is accumulated from the same fp32 products in the same order, A and B come out
// exactly symmetric here as well.
#include "muon_internal.h"

namespace muon {
namespace {

constexpr int TM = 64, TK = 16;

enum Mode { GRAM = 0, POLY = 1, APPLY = 2 };

struct GemmArgsF {
  const float* lhs;  // [batch][M][K]
  const float* rhs;  // GRAM/POLY: [batch][N][K]; APPLY: [batch][K][N]
  const float* epi;  // POLY: A, APPLY: X (laid out like out)
  float* out;        // [batch][M][N]
  long long lhs_bs, rhs_bs, out_bs;
  int ld_lhs, ld_rhs, ld_out;
  int K, tiles_n;
  const float* scales;
  int scale_idx;
  float alpha, beta;
};

template <int MODE>
__global__ __launch_bounds__(256) void ns_gemm_f32(GemmArgsF g) {
  __shared__ float sA[TK][TM + 4];
  __shared__ float sB[TK][TM + 4];
  const int t = threadIdx.x;
  const int tx = t & 15, ty = t >> 4;
  const int bidx = blockIdx.y;
  const int I = blockIdx.x / g.tiles_n, J = blockIdx.x % g.tiles_n;
  const float* lhs = g.lhs + bidx * g.lhs_bs + (size_t)(I * TM) * g.ld_lhs;
  const float* rhs = g.rhs + bidx * g.rhs_bs +
                     (MODE == APPLY ? (size_t)(J * TM) : (size_t)(J * TM) * g.ld_rhs);
  float acc[4][4] = {};

  for (int k0 = 0; k0 < g.K; k0 += TK) {
    {  // lhs tile: 64 rows x 16 k, one float4 along k per thread, stored k-major
      const int r = t >> 2, kk = 4 * (t & 3);
      const float4 v = *reinterpret_cast<const float4*>(lhs + (size_t)r * g.ld_lhs + k0 + kk);
      sA[kk + 0][r] = v.x; sA[kk + 1][r] = v.y; sA[kk + 2][r] = v.z; sA[kk + 3][r] = v.w;
    }
    if (MODE == APPLY) {  // rhs tile: 16 k-rows x 64 n, already k-major
      const int kk = t >> 4, n = 4 * (t & 15);
      const float4 v = *reinterpret_cast<const float4*>(rhs + (size_t)(k0 + kk) * g.ld_rhs + n);
      sB[kk][n + 0] = v.x; sB[kk][n + 1] = v.y; sB[kk][n + 2] = v.z; sB[kk][n + 3] = v.w;
    } else {              // rhs tile: 64 n-rows x 16 k, transposed into k-major
      const int n = t >> 2, kk = 4 * (t & 3);
      const float4 v = *reinterpret_cast<const float4*>(rhs + (size_t)n * g.ld_rhs + k0 + kk);
      sB[kk + 0][n] = v.x; sB[kk + 1][n] = v.y; sB[kk + 2][n] = v.z; sB[kk + 3][n] = v.w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

  const float s = g.scales ? g.scales[4 * bidx + g.scale_idx] : 1.f;
  float* out = g.out + bidx * g.out_bs;
  const float* epi = (MODE == GRAM) ? nullptr : g.epi + bidx * g.out_bs;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gi = I * TM + ty + 16 * i, gj = J * TM + tx + 16 * j;
      const size_t o = (size_t)gi * g.ld_out + gj;
      float v;
      if (MODE == GRAM) v = acc[i][j] * s;
      else if (MODE == POLY) v = fmaf(g.alpha, epi[o], g.beta * acc[i][j]);
      else v = fmaf(g.alpha, epi[o], acc[i][j]) * s;
      out[o] = v;
    }
  }
}

}  // namespace

hipError_t launch_gram_f32(const NsGroup& G, hipStream_t s) {
  GemmArgsF a{};
  a.lhs = a.rhs = static_cast<const float*>(G.x_in);
  a.out = static_cast<float*>(G.a);
  a.lhs_bs = a.rhs_bs = (long long)G.mp * G.np;
  a.out_bs = (long long)G.mp * G.mp;
  a.ld_lhs = a.ld_rhs = G.np;
  a.ld_out = G.mp;
  a.K = G.np;
  a.tiles_n = G.mp / TM;
  a.scales = G.first ? G.scales : nullptr;
  a.scale_idx = 1;
  launch_k(ns_gemm_f32<GRAM>, dim3((G.mp / TM) * (G.mp / TM), G.batch), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

hipError_t launch_poly_f32(const NsGroup& G, float b, float c, hipStream_t s) {
  GemmArgsF a{};
  a.lhs = a.rhs = a.epi = static_cast<const float*>(G.a);
  a.out = static_cast<float*>(G.b);
  a.lhs_bs = a.rhs_bs = a.out_bs = (long long)G.mp * G.mp;
  a.ld_lhs = a.ld_rhs = a.ld_out = G.mp;
  a.K = G.mp;
  a.tiles_n = G.mp / TM;
  a.alpha = b;
  a.beta = c;
  launch_k(ns_gemm_f32<POLY>, dim3((G.mp / TM) * (G.mp / TM), G.batch), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

hipError_t launch_apply_f32(const NsGroup& G, float alpha, hipStream_t s) {
  GemmArgsF a{};
  a.lhs = static_cast<const float*>(G.b);
  a.rhs = a.epi = static_cast<const float*>(G.x_in);
  a.out = static_cast<float*>(G.x_out);
  a.lhs_bs = (long long)G.mp * G.mp;
  a.rhs_bs = a.out_bs = (long long)G.mp * G.np;
  a.ld_lhs = G.mp;
  a.ld_rhs = a.ld_out = G.np;
  a.K = G.mp;
  a.tiles_n = G.np / TM;
  a.scales = G.first ? G.scales : nullptr;
  a.scale_idx = 0;
  a.alpha = alpha;
  launch_k(ns_gemm_f32<APPLY>, dim3((G.mp / TM) * (G.np / TM), G.batch), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace muon
