// Offline packer on the GPU: dense expert weights in, the stored form of one
// projection out (the input of tq_upload_proj).
//
// "TileQ" technical summary, section 2.1 step 4: the K experts are tiles of
// one block matrix W_big on the M x N grid (a tile without an expert is a zero
// block); step 5: W_big gets a global low-rank decomposition U Sigma V^T
// approximated by Gaussian sketching instead of a full SVD, the factors are
// stored, and each expert's residual is quantized.
//
// The sketch is the randomized range finder with a small SVD, all in fp64:
//   Y = W_big Omega                                (Omega [n][l] given)
//   Q = Y T, T = P diag(lambda^-1/2) from the eigendecomposition of Y^T Y
//       (directions with lambda below 1e-13 lambda_max dropped), done twice
//   power iterations: Y = W_big (W_big^T Q), orthonormalised again
//   Z = W_big^T Q  (= B^T, B = Q^T W_big)
//   Z^T Z = B B^T = U~ diag(s^2) U~^T (eigendecomposition, descending)
//   U = Q U~_r, sigma = s_r, V = Z U~_r diag(1 / s_r)
// The factors are stored as U, V in the activation format and sigma in fp32;
// each expert's residual W_e - U_m diag(sigma) V_n^T is taken against those
// stored values and quantized by asymmetric round to nearest per group of G
// inputs (the forward's residual format): s = RND_f16((mx - mn) / Q) with
// mn = min(min w, 0), mx = max(max w, 0) (1 when 0), z = clamp(rint(-mn / s)),
// q = clamp(rint(w / s) + z), in fp64.
//
// Kernels: an LDS-tiled fp64 GEMM with operand readers for W_big (gathered
// from the expert tiles, converted from the weights' dtype on load), its
// transpose and dense arrays (split-K into slabs for the Gram matrices); a
// one-workgroup cyclic Jacobi eigensolver for the l x l symmetric matrices
// (l <= 136, the matrix in LDS); small elementwise kernels; the residual
// quantizer that packs the codes.  fp64 runs on the vector ALUs: on gfx950 the
// fp64 matrix rate equals the vector rate.
#include "tq_device.h"

namespace tq {

constexpr int PK_T = 256;      // threads per workgroup
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int PK_TM = 64, PK_TN = 64, PK_TK = 16;
constexpr int PK_LMAX = 136;   // largest sketch width (rank 128 + 8)

// value of the weights' storage type as fp64 (WDT 0 f16, 1 bf16, 2 f32, 3 f64)
template <int WDT>
__device__ __forceinline__ double w_at(const void* W, size_t idx) {
  if constexpr (WDT == 0) return (double)(float)reinterpret_cast<const half_t*>(W)[idx];
  else if constexpr (WDT == 1)
    return (double)__uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(W)[idx] << 16);
  else if constexpr (WDT == 2) return (double)reinterpret_cast<const float*>(W)[idx];
  else return reinterpret_cast<const double*>(W)[idx];
}

// eight consecutive weights (16-byte aligned for 2-byte types) as fp64
template <int WDT>
__device__ __forceinline__ void w_at8(const void* W, size_t idx, double* v) {
  if constexpr (WDT == 0 || WDT == 1) {
    const uint4 q = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(W) + idx);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint16_t h = (uint16_t)(w[u >> 1] >> (16 * (u & 1)));
      if constexpr (WDT == 0) v[u] = (double)(float)__builtin_bit_cast(half_t, h);
      else v[u] = (double)__uint_as_float((uint32_t)h << 16);
    }
  } else if constexpr (WDT == 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float4 q = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(W) + idx + 4 * h);
      v[4 * h] = q.x;
      v[4 * h + 1] = q.y;
      v[4 * h + 2] = q.z;
      v[4 * h + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const double2 q = *reinterpret_cast<const double2*>(reinterpret_cast<const double*>(W) + idx + 2 * h);
      v[2 * h] = q.x;
      v[2 * h + 1] = q.y;
    }
  }
}

enum { AM_DENSE = 0, AM_DENSE_T = 1, AM_WBIG = 2, AM_WBIG_T = 3 };
enum { BM_DENSE = 0, BM_DENSE_T = 1 };

struct PkGemm {
  int M, N, K;
  const double* A;
  int lda;
  const void* W;                 // AM_WBIG(_T): expert weights [K][d_out][d_in], dtype wdt
  int wdt, d_out, d_in, Ng;      // Ng: grid columns
  const int* emap;               // [Mg * Ng] expert at each tile, -1 for an empty tile
  const double* B;
  int ldb;
  double* C;
  int ldc;
  size_t slab;                   // split-K: slab z at C + z * slab
  int kchunk;                    // split-K: K range of one slab (multiple of the kernel's TK)
};

// C[i][j] = sum_k A(i, k) B(k, j) over this slab's K range.  Tiles of 64 rows
// x 16 NC columns (NC = 4: several column tiles; NC = 5 or 9: one tile of up
// to 80 or 144 columns, the sketch's width), each thread 4 rows x NC columns,
// K in chunks of 16 staged through LDS, the next chunk's loads in flight
// during the current chunk's arithmetic.  W_big readers: a chunk of 16 k never
// crosses a tile (d_in % 128 == 0, d_out % 16 == 0), so the tile and its
// expert are found once per chunk and row (no division per element).
// TK: the K chunk, 16, or 32 for the W_big readers when every chunk stays
// inside one tile: then each thread reads eight consecutive weights of one
// row with one 16-byte load (the 2-byte weights would otherwise take one
// load instruction each).
template <int AM, int BM, int NC, int WDT, int TK = PK_TK>
__global__ __launch_bounds__(PK_T) void pk_gemm_kernel(PkGemm g) {
  constexpr int TN = 16 * NC;
  constexpr bool WV = (AM == AM_WBIG || AM == AM_WBIG_T) && TK == 32;   // vector W loads
  static_assert(TK == 16 || WV, "32-input chunks for the W_big readers only");
  constexpr int TM = WV ? 2 * PK_TM : PK_TM;      // rows of the tile (W_big: 128, fewer B reads)
  constexpr int NA = WV ? 16 : 4;                // A values per thread and chunk
  constexpr int NB = NC * TK / 16;               // B values per thread and chunk
  __shared__ double sA[TK][TM + 2];
  __shared__ double sB[TK][TN + 2];
  const int tid = threadIdx.x;
  const int i0 = blockIdx.y * TM, j0 = blockIdx.x * TN;
  const int k_begin = blockIdx.z * g.kchunk;
  const int k_end = min(g.K, k_begin + g.kchunk);
  const int ty = tid >> 4, tx = tid & 15;
  // W_big readers: the parts of the address fixed for the whole kernel
  //   AM_WBIG:   rows i = (tid >> 4) + 16 s (4 per thread): tile row and row in tile
  //   AM_WBIG_T: column i = tid & 63 of A is a column of W_big: tile column, input
  int rt_m[4] = {0, 0, 0, 0}, rt_o[4] = {0, 0, 0, 0};
  int ct_n = 0, ct_i = 0;
  if constexpr (WV && AM == AM_WBIG) {
    // rows i = (tid >> 2) + 64 h (h = 0, 1), inputs 8 (tid & 3) .. + 7 of the chunk
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int gi = min(i0 + (tid >> 2) + 64 * h, g.M - 1);
      rt_m[h] = gi / g.d_out;
      rt_o[h] = gi - rt_m[h] * g.d_out;
    }
  } else if constexpr (WV && AM == AM_WBIG_T) {
    // columns i0 + 8 (tid & 15) .. + 7 of W_big (one tile column), rows
    // (tid >> 4) + 16 h of the chunk
    const int gi = min(i0 + 8 * (tid & 15), g.M - 1);
    ct_n = gi / g.d_in;
    ct_i = gi - ct_n * g.d_in;
  } else if constexpr (AM == AM_WBIG) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int gi = min(i0 + (tid >> 4) + 16 * s, g.M - 1);
      rt_m[s] = gi / g.d_out;
      rt_o[s] = gi - rt_m[s] * g.d_out;
    }
  } else if constexpr (AM == AM_WBIG_T) {
    const int gi = min(i0 + (tid & 63), g.M - 1);
    ct_n = gi / g.d_in;
    ct_i = gi - ct_n * g.d_in;
  }
  // A and B values of a K chunk, loaded into registers one chunk ahead of
  // the arithmetic (the global loads of chunk k0 + 16 are in flight while
  // chunk k0 is multiplied from LDS)
  double ra[NA], rb[NB];
  auto load_chunk = [&](int k0) {
    if constexpr (WV && AM == AM_WBIG) {
      const int nt = k0 / g.d_in, q = tid & 3;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int i = (tid >> 2) + 64 * h;
        const int e = (i0 + i < g.M && k0 + 8 * q < k_end) ? g.emap[rt_m[h] * g.Ng + nt] : -1;
        if (e >= 0) {
          w_at8<WDT>(g.W, ((size_t)e * g.d_out + rt_o[h]) * g.d_in + (k0 - nt * g.d_in) + 8 * q,
                     ra + 8 * h);
        } else {
#pragma unroll
          for (int u = 0; u < 8; ++u) ra[8 * h + u] = 0.0;
        }
      }
    } else if constexpr (WV && AM == AM_WBIG_T) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kk = (tid >> 4) + 16 * h;
        const int mt = (k0 + kk) / g.d_out, o = k0 + kk - mt * g.d_out;
        const int e = (i0 + 8 * (tid & 15) < g.M && k0 + kk < k_end) ? g.emap[mt * g.Ng + ct_n] : -1;
        if (e >= 0) {
          w_at8<WDT>(g.W, ((size_t)e * g.d_out + o) * g.d_in + ct_i, ra + 8 * h);
        } else {
#pragma unroll
          for (int u = 0; u < 8; ++u) ra[8 * h + u] = 0.0;
        }
      }
    } else if constexpr (AM == AM_WBIG) {
      const int nt = k0 / g.d_in, ii0 = k0 - nt * g.d_in;
      const int kk = tid & 15;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int i = (tid >> 4) + 16 * s;
        double v = 0.0;
        if (i0 + i < g.M && k0 + kk < k_end) {
          const int e = g.emap[rt_m[s] * g.Ng + nt];
          if (e >= 0) v = w_at<WDT>(g.W, ((size_t)e * g.d_out + rt_o[s]) * g.d_in + ii0 + kk);
        }
        ra[s] = v;
      }
    } else if constexpr (AM == AM_WBIG_T) {
      const int mt = k0 / g.d_out, o0 = k0 - mt * g.d_out;
      const int e = g.emap[mt * g.Ng + ct_n];
      const int i = tid & 63;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int kk = (tid >> 6) + 4 * s;
        double v = 0.0;
        if (i0 + i < g.M && k0 + kk < k_end && e >= 0)
          v = w_at<WDT>(g.W, ((size_t)e * g.d_out + o0 + kk) * g.d_in + ct_i);
        ra[s] = v;
      }
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        int i, kk;
        if constexpr (AM == AM_DENSE) {
          kk = tid & 15;
          i = (tid >> 4) + 16 * s;
        } else {
          i = tid & 63;
          kk = (tid >> 6) + 4 * s;
        }
        const int gi = i0 + i, gk = k0 + kk;
        double v = 0.0;
        if (gi < g.M && gk < k_end) {
          if constexpr (AM == AM_DENSE) v = g.A[(size_t)gi * g.lda + gk];
          else v = g.A[(size_t)gk * g.lda + gi];
        }
        ra[s] = v;
      }
    }
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const int idx = tid + PK_T * t;            // TK TN = 256 NB elements
      int j, kk;
      if constexpr (BM == BM_DENSE) {
        j = idx % TN;
        kk = idx / TN;
      } else {
        kk = idx & 15;
        j = idx >> 4;
      }
      const int gj = j0 + j, gk = k0 + kk;
      double v = 0.0;
      if (gj < g.N && gk < k_end) {
        if constexpr (BM == BM_DENSE) v = g.B[(size_t)gk * g.ldb + gj];
        else v = g.B[(size_t)gj * g.ldb + gk];
      }
      rb[t] = v;
    }
  };
  auto store_chunk = [&]() {
    if constexpr (WV && AM == AM_WBIG) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int u = 0; u < 8; ++u) sA[8 * (tid & 3) + u][(tid >> 2) + 64 * h] = ra[8 * h + u];
    } else if constexpr (WV && AM == AM_WBIG_T) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int u = 0; u < 8; ++u) sA[(tid >> 4) + 16 * h][8 * (tid & 15) + u] = ra[8 * h + u];
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if constexpr (AM == AM_DENSE || AM == AM_WBIG) sA[tid & 15][(tid >> 4) + 16 * s] = ra[s];
        else sA[(tid >> 6) + 4 * s][tid & 63] = ra[s];
      }
    }
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const int idx = tid + PK_T * t;
      if constexpr (BM == BM_DENSE) sB[idx / TN][idx % TN] = rb[t];
      else sB[idx & 15][idx >> 4] = rb[t];
    }
  };
  // The W_big products run on the fp64 matrix cores: wave w takes rows
  // 32 w .. 32 w + 31 of the tile (two row tiles) against all NC column tiles,
  // v_mfma_f64_16x16x4f64 per 4 k (lane l: A[l % 16][l / 16], B[l / 16][l % 16];
  // result element j of lane l at row 4 j + l / 16, column l % 16).  Other
  // products: 4 x NC fp64 FMAs per thread.
  constexpr bool MF = WV;
  double acc[4][NC] = {};
  f64x4 macc[MF ? 2 : 1][MF ? NC : 1];
#pragma unroll
  for (int r = 0; r < (MF ? 2 : 1); ++r)
#pragma unroll
    for (int v = 0; v < (MF ? NC : 1); ++v) macc[r][v] = f64x4{0.0, 0.0, 0.0, 0.0};
  const int lane = tid & 63, wv = tid >> 6;
  if (k_begin < k_end) load_chunk(k_begin);
  for (int k0 = k_begin; k0 < k_end; k0 += TK) {
    store_chunk();
    __syncthreads();
    if (k0 + TK < k_end) load_chunk(k0 + TK);
    if constexpr (MF) {
#pragma unroll
      for (int k4 = 0; k4 < TK; k4 += 4) {
        double b[NC];
#pragma unroll
        for (int v = 0; v < NC; ++v) b[v] = sB[k4 + (lane >> 4)][16 * v + (lane & 15)];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const double a = sA[k4 + (lane >> 4)][32 * wv + 16 * r + (lane & 15)];
#pragma unroll
          for (int v = 0; v < NC; ++v)
            macc[r][v] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b[v], macc[r][v], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < TK; ++kk) {
        double a[4], b[NC];
#pragma unroll
        for (int u = 0; u < 4; ++u) a[u] = sA[kk][ty * 4 + u];
#pragma unroll
        for (int v = 0; v < NC; ++v) b[v] = sB[kk][tx + 16 * v];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = 0; v < NC; ++v) acc[u][v] = fma(a[u], b[v], acc[u][v]);
      }
    }
    __syncthreads();
  }
  double* C = g.C + (size_t)blockIdx.z * g.slab;
  if constexpr (MF) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int v = 0; v < NC; ++v) {
        const int gj = j0 + 16 * v + (lane & 15);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int gi = i0 + 32 * wv + 16 * r + 4 * j + (lane >> 4);
          if (gi < g.M && gj < g.N) C[(size_t)gi * g.ldc + gj] = macc[r][v][j];
        }
      }
    return;
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int gi = i0 + ty * 4 + u;
    if (gi >= g.M) continue;
#pragma unroll
    for (int v = 0; v < NC; ++v) {
      const int gj = j0 + tx + 16 * v;
      if (gj < g.N) C[(size_t)gi * g.ldc + gj] = acc[u][v];
    }
  }
}

// K range of one split-K slab and the number of slabs for `splits` requested
static int pk_kchunk(int K, int splits, int tk = PK_TK) {
  splits = std::max(1, splits);
  return std::max(tk, ((K + splits - 1) / splits + tk - 1) / tk * tk);
}
static int pk_nslab(int K, int splits, int tk = PK_TK) {
  const int kc = pk_kchunk(K, splits, tk);
  return std::max(1, (K + kc - 1) / kc);
}
// K chunk of a product: 32 for the W_big readers whose chunks stay inside a
// tile (along d_in always; along d_out when it is a multiple of 32)
static int pk_tk(const PkGemm& g, int amode) {
  if (amode == AM_WBIG) return 32;
  if (amode == AM_WBIG_T && g.d_out % 32 == 0) return 32;
  return PK_TK;
}

template <int AM, int BM, int NC, int TK>
static void pk_launch_wdt(const PkGemm& g, dim3 grid, hipStream_t s) {
  switch (g.wdt) {
    case 0: hipLaunchKernelGGL((pk_gemm_kernel<AM, BM, NC, 0, TK>), grid, dim3(PK_T), 0, s, g); break;
    case 1: hipLaunchKernelGGL((pk_gemm_kernel<AM, BM, NC, 1, TK>), grid, dim3(PK_T), 0, s, g); break;
    case 2: hipLaunchKernelGGL((pk_gemm_kernel<AM, BM, NC, 2, TK>), grid, dim3(PK_T), 0, s, g); break;
    default: hipLaunchKernelGGL((pk_gemm_kernel<AM, BM, NC, 3, TK>), grid, dim3(PK_T), 0, s, g); break;
  }
}

template <int AM, int BM, int NC>
static void pk_launch_w(const PkGemm& g, dim3 grid, hipStream_t s) {
  if constexpr (AM == AM_WBIG || AM == AM_WBIG_T) {
    if (pk_tk(g, AM) == 32) pk_launch_wdt<AM, BM, NC, 32>(g, grid, s);
    else pk_launch_wdt<AM, BM, NC, PK_TK>(g, grid, s);
  } else {
    hipLaunchKernelGGL((pk_gemm_kernel<AM, BM, NC, 3>), grid, dim3(PK_T), 0, s, g);
  }
}

template <int NC>
static void pk_launch_nc(const PkGemm& g, int amode, int bmode, dim3 grid, hipStream_t s) {
  if (bmode == BM_DENSE_T) {
    pk_launch_w<AM_DENSE, BM_DENSE_T, NC>(g, grid, s);
    return;
  }
  switch (amode) {
    case AM_DENSE: pk_launch_w<AM_DENSE, BM_DENSE, NC>(g, grid, s); break;
    case AM_DENSE_T: pk_launch_w<AM_DENSE_T, BM_DENSE, NC>(g, grid, s); break;
    case AM_WBIG: pk_launch_w<AM_WBIG, BM_DENSE, NC>(g, grid, s); break;
    default: pk_launch_w<AM_WBIG_T, BM_DENSE, NC>(g, grid, s); break;
  }
}

// out[i] = sum over slabs z of C[z * slab + i] (slab order fixed: deterministic)
__global__ void pk_sum_slabs_kernel(const double* __restrict__ C, int nslab, size_t slab, size_t count,
                                    double* __restrict__ out) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (size_t)gridDim.x * blockDim.x) {
    double v = 0.0;
    for (int z = 0; z < nslab; ++z) v += C[z * slab + i];
    out[i] = v;
  }
}

void launch_pk_gemm(const PkGemm& g0, int amode, int bmode, int splits, hipStream_t s) {
  PkGemm g = g0;
  const int tk = pk_tk(g, amode);
  g.kchunk = pk_kchunk(g.K, splits, tk);
  splits = pk_nslab(g.K, splits, tk);
  // one column tile for the sketch's widths (up to 144), else tiles of 64
  const int nc = (g.N <= 64) ? 4 : (g.N <= 80 ? 5 : (g.N <= 144 ? 9 : 4));
  const int tm = (tk == 32) ? 2 * PK_TM : PK_TM;   // rows per tile (as the kernel's TM)
  const dim3 grid((g.N + 16 * nc - 1) / (16 * nc), (g.M + tm - 1) / tm, std::max(1, splits));
  if (nc == 5) pk_launch_nc<5>(g, amode, bmode, grid, s);
  else if (nc == 9) pk_launch_nc<9>(g, amode, bmode, grid, s);
  else pk_launch_nc<4>(g, amode, bmode, grid, s);
}

// The same product into `out` (ldc = N) through `splits` split-K slabs at
// `slabs` ([splits][M][N]) summed in slab order: more workgroups for the
// long-K products of W_big.
static void launch_pk_gemm_split(const PkGemm& g0, int amode, int splits, double* slabs, double* out,
                                 hipStream_t s) {
  PkGemm g = g0;
  g.C = slabs;
  g.ldc = g.N;
  g.slab = (size_t)g.M * g.N;
  launch_pk_gemm(g, amode, BM_DENSE, splits, s);
  const int nslab = pk_nslab(g.K, splits, pk_tk(g, amode));
  const size_t count = (size_t)g.M * g.N;
  hipLaunchKernelGGL(pk_sum_slabs_kernel, dim3((unsigned)std::min<size_t>((count + 255) / 256, 8192)),
                     dim3(256), 0, s, slabs, nslab, g.slab, count, out);
}

// ---- symmetric eigendecomposition of an l x l matrix (one workgroup) -------
// The matrix is the sum of `nslab` slabs (split-K partial Gram matrices) of
// which the upper triangle is read.  Cyclic Jacobi with the round-robin
// (circle) ordering: each round rotates l/2 disjoint pairs (p, q) at once --
// rows of A, then columns of A and rows of the transposed eigenvector matrix
// E^T (in LDS for l <= 96, else global memory) -- and a sweep is l - 1
// rounds; sweeps stop when the off-diagonal mass is below `tol` of the total
// (1e-24: off-diagonal entries ~1e-12 of the matrix, eigenvalues to ~1e-24,
// vectors to ~1e-12), or when a sweep no longer halves it (the rounding
// floor), at most 40.  The rotation for a pair zeroes a_pq:
// theta = (a_qq - a_pp) / (2 a_pq), t = sign(theta) / (|theta| + sqrt(theta^2 + 1)),
// c = 1 / sqrt(t^2 + 1), s = t c.  Output: eigenvalues descending in eval,
// eigenvector j in column j of evec (ties in index order).
// Rows of A and E^T are `ld` = l | 1 doubles apart: an odd stride keeps a
// column walk (one row per lane) free of LDS bank conflicts.
// LM: the largest l of the instance; ELDS: E in LDS too (l <= 96), else in
// global memory (l x ld doubles at Eg).
constexpr int PK_JT = 1024;    // threads of the eigensolver's workgroup

template <int LM, bool ELDS>
__global__ __launch_bounds__(PK_JT) void pk_jacobi_kernel(const double* __restrict__ G, int l,
                                                         int nslab, size_t slab,
                                                         double* __restrict__ Eg,
                                                         double* __restrict__ evec,
                                                         double* __restrict__ eval, double tol) {
  constexpr int LDM = LM | 1;
  __shared__ double sA[LM * LDM];
  __shared__ double sE[ELDS ? LM * LDM : 1];
  __shared__ double s_c[LM / 2 + 1], s_s[LM / 2 + 1];
  __shared__ int s_p[LM / 2 + 1], s_q[LM / 2 + 1];
  double* const Et = ELDS ? sE : Eg;
  __shared__ double s_red[PK_JT / 64][2];
  __shared__ int s_stop;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ld = l | 1;
  for (int idx = tid; idx < l * l; idx += PK_JT) {
    const int a = idx / l, b = idx - a * l;
    const int r0 = min(a, b), c0 = max(a, b);
    double v = 0.0;
    for (int z = 0; z < nslab; ++z) v += G[z * slab + (size_t)r0 * l + c0];
    sA[a * ld + b] = v;
    Et[(size_t)a * ld + b] = (a == b) ? 1.0 : 0.0;
  }
  __syncthreads();
  const int le = l + (l & 1);          // even number of players (one dummy when l is odd)
  const int np = le / 2;
  // this thread's (pair, index) work items of a round, the same every round
  constexpr int NW = (LM / 2 * LM + PK_JT - 1) / PK_JT;
  int wk[NW], wj[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int idx = tid + PK_JT * w;
    wk[w] = idx / l;
    wj[w] = idx - wk[w] * l;
  }
  double prev_off = -1.0;              // (thread 0) off-diagonal mass of the previous sweep
  for (int sweep = 0; sweep < 40; ++sweep) {
    // convergence: off-diagonal against total squared mass
    double off = 0.0, tot = 0.0;
    for (int idx = tid; idx < l * l; idx += PK_JT) {
      const int a = idx / l, b = idx - a * l;
      const double v = sA[a * ld + b];
      tot += v * v;
      if (a != b) off += v * v;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      off += __shfl_xor(off, o, 64);
      tot += __shfl_xor(tot, o, 64);
    }
    if (lane == 0) {
      s_red[wv][0] = off;
      s_red[wv][1] = tot;
    }
    __syncthreads();
    if (tid == 0) {
      double o2 = 0.0, t2 = 0.0;
      for (int w = 0; w < PK_JT / 64; ++w) {
        o2 += s_red[w][0];
        t2 += s_red[w][1];
      }
      // converged, or at the rounding floor (the last sweep did not halve it)
      s_stop = (o2 <= tol * t2 || (prev_off >= 0.0 && o2 > 0.5 * prev_off)) ? 1 : 0;
      prev_off = o2;
    }
    __syncthreads();
    if (s_stop) break;
    for (int round = 0; round < le - 1; ++round) {
      // circle method: player 0 fixed, the others rotate
      if (tid < np) {
        // (x - 1 + round < 2 (le - 1): the remainder is one conditional subtraction)
        auto pos = [&](int x) {
          const int t = x - 1 + round;
          return x == 0 ? 0 : 1 + (t >= le - 1 ? t - (le - 1) : t);
        };
        const int a0 = pos(tid), b0 = pos(le - 1 - tid);
        const int p = min(a0, b0), q = max(a0, b0);
        double c = 1.0, sn = 0.0;
        if (q < l) {
          const double apq = sA[p * ld + q];
          if (apq != 0.0) {
            const double theta = (sA[q * ld + q] - sA[p * ld + p]) / (2.0 * apq);
            const double t = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
            c = 1.0 / sqrt(t * t + 1.0);
            sn = t * c;
          }
        }
        s_p[tid] = p;
        s_q[tid] = (q < l) ? q : -1;             // -1: the dummy player, no rotation
        s_c[tid] = c;
        s_s[tid] = sn;
      }
      __syncthreads();
      // rows p, q of A (J^T A) and of E^T (J^T E^T = (E J)^T)
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int idx = tid + PK_JT * w;
        if (idx >= np * l) continue;
        const int k = wk[w], j = wj[w];
        const int p = s_p[k], q = s_q[k];
        if (q < 0) continue;
        const double c = s_c[k], sn = s_s[k];
        const double ap = sA[p * ld + j], aq = sA[q * ld + j];
        sA[p * ld + j] = c * ap - sn * aq;
        sA[q * ld + j] = sn * ap + c * aq;
        const double ep = Et[(size_t)p * ld + j], eq = Et[(size_t)q * ld + j];
        Et[(size_t)p * ld + j] = c * ep - sn * eq;
        Et[(size_t)q * ld + j] = sn * ep + c * eq;
      }
      __syncthreads();
      // columns p, q of A (A J)
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int idx = tid + PK_JT * w;
        if (idx >= np * l) continue;
        const int k = wk[w], j = wj[w];
        const int p = s_p[k], q = s_q[k];
        if (q < 0) continue;
        const double c = s_c[k], sn = s_s[k];
        const double ap = sA[j * ld + p], aq = sA[j * ld + q];
        sA[j * ld + p] = c * ap - sn * aq;
        sA[j * ld + q] = sn * ap + c * aq;
      }
      if constexpr (!ELDS) __threadfence_block();
      __syncthreads();
    }
  }
  // descending order: rank of eigenvalue j (ties by index)
  for (int j = tid; j < l; j += PK_JT) {
    const double v = sA[j * ld + j];
    int rank = 0;
    for (int i = 0; i < l; ++i) {
      const double w = sA[i * ld + i];
      rank += (w > v || (w == v && i < j)) ? 1 : 0;
    }
    eval[rank] = v;
    for (int a = 0; a < l; ++a) evec[(size_t)a * l + rank] = Et[(size_t)j * ld + a];
  }
}

static void launch_pk_jacobi(const double* G, int l, int nslab, size_t slab, double* E, double* evec,
                             double* eval, double tol, hipStream_t s) {
  if (l <= 96)
    hipLaunchKernelGGL((pk_jacobi_kernel<96, true>), dim3(1), dim3(PK_JT), 0, s, G, l, nslab, slab, E,
                       evec, eval, tol);
  else
    hipLaunchKernelGGL((pk_jacobi_kernel<PK_LMAX, false>), dim3(1), dim3(PK_JT), 0, s, G, l, nslab,
                       slab, E, evec, eval, tol);
}

// T[a][j] = evec[a][j] / sqrt(eval[j]) for eval[j] > rel * eval[0], else 0
// (orthonormalisation transform of a basis from its Gram matrix)
__global__ void pk_whiten_kernel(const double* __restrict__ evec, const double* __restrict__ eval,
                                 int l, double rel, double* __restrict__ T) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= l * l) return;
  const int j = idx % l;
  const double lam = eval[j], top = eval[0];
  T[idx] = (top > 0.0 && lam > rel * top) ? evec[idx] / sqrt(lam) : 0.0;
}

// The leading r columns of U~ scaled for V: S[a][c] = evec[a][c] / s_c with
// s_c = sqrt(eval[c]) (0 where s_c is 0), and sigma64[c] = s_c.
__global__ void pk_vscale_kernel(const double* __restrict__ evec, const double* __restrict__ eval,
                                 int l, int r, double* __restrict__ Sv, double* __restrict__ sig64) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= l * r) return;
  const int a = idx / r, c = idx - a * r;
  const double sv = sqrt(fmax(eval[c], 0.0));
  Sv[idx] = (sv > 0.0) ? evec[(size_t)a * l + c] / sv : 0.0;
  if (a == 0) sig64[c] = sv;
}

// fp64 -> fp16 / bf16 bits, one rounding to nearest even (the format's grid:
// 11 or 8 significant bits, smallest normal exponent -14 or -126, quantum
// 2^-24 or 2^-133 below it; overflow to infinity)
__device__ __forceinline__ uint16_t rnd_f64_to(double v, int bf) {
  const int bits = bf ? 8 : 11, emin = bf ? -126 : -14;
  const double vmax = bf ? 3.3895313892515355e38 : 65504.0;
  const uint16_t sign = signbit(v) ? 0x8000u : 0u;
  const double a = fabs(v);
  if (a == 0.0) return sign;
  int ex;
  frexp(a, &ex);                                   // a = m 2^ex, m in [0.5, 1)
  const int qexp = max(ex - 1, emin) - (bits - 1);
  const double r = ldexp(rint(ldexp(a, -qexp)), qexp);
  const double limit = vmax + ldexp(1.0, (bf ? 127 : 15) - bits);   // halfway above vmax
  if (a >= limit) return sign | (bf ? 0x7F80u : 0x7C00u);
  // r is exactly representable: take its fp32 bits (bf16 = high half; fp16 by conversion)
  const float rf = (float)r;
  if (bf) return sign | (uint16_t)(__float_as_uint(rf) >> 16);
  return sign | (uint16_t)__builtin_bit_cast(uint16_t, (half_t)rf);
}

// U or V columns 0..r-1 from an fp64 [rows][ld] array to the activation format
// [rows][r]; and the fp64 values of the stored numbers (times sigma32 when
// given) for the residual.
__global__ void pk_store_kernel(const double* __restrict__ X, int rows, int ld, int r, int bf,
                                uint16_t* __restrict__ out, const float* __restrict__ sig32,
                                double* __restrict__ x64) {
  const size_t total = (size_t)rows * r;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const size_t i = idx / r;
    const int c = (int)(idx - i * r);
    const uint16_t h = rnd_f64_to(X[i * ld + c], bf);
    out[idx] = h;
    const double v = bf ? (double)__uint_as_float((uint32_t)h << 16)
                        : (double)(float)__builtin_bit_cast(half_t, h);
    x64[idx] = sig32 ? v * (double)sig32[c] : v;
  }
}

__global__ void pk_sigma_kernel(const double* __restrict__ sig64, int r, float* __restrict__ sig32) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c < r) sig32[c] = (float)sig64[c];
}

// Residual of expert e, w = W_e[o][i] - L[o][i] (L its block of the stored
// low-rank product), quantized per group.  One thread per 32 consecutive
// inputs of a row (the residual kept in registers); the LPG = G / 32 threads
// of a group (a power of two, aligned inside a wave) meet by xor shuffles for
// the group's min and max; each thread packs its 32 codes into its own words
// (2-bit: 2 words, code i at bits 2 (i % 16); 3-bit: 3 words of the row's bit
// string).  LPG = 0: any G, one thread per group looping over it.
template <int LPG, int WDT>
__global__ __launch_bounds__(256) void pk_rtn_kernel(const void* __restrict__ W, int e, int d_out,
                                                     int d_in, int G, int bits,
                                                     const double* __restrict__ L,
                                                     uint32_t* __restrict__ codes,
                                                     uint16_t* __restrict__ scales,
                                                     uint16_t* __restrict__ zeros) {
  const int qmax = (1 << bits) - 1;
  const int ng = d_in / G;
  const size_t wpr = (size_t)bits * d_in / 32;                 // code words per row
  auto finish_scale = [&](double mn, double mx, double* s, double* z, int o, int g) {
    const uint16_t sb = rnd_f64_to((mx - mn) / (double)qmax, 0);
    double sv = (double)(float)__builtin_bit_cast(half_t, sb);
    uint16_t sbits = sb;
    if (sv == 0.0) {
      sv = 1.0;
      sbits = 0x3C00u;
    }
    *s = sv;
    *z = fmin(fmax(rint(-mn / sv), 0.0), (double)qmax);
    const size_t sz = ((size_t)e * d_out + o) * ng + g;
    scales[sz] = sbits;
    zeros[sz] = __builtin_bit_cast(uint16_t, (half_t)(float)*z);
  };
  // the 32 codes of inputs c0 .. c0 + 31 of row o into the row's words
  auto emit = [&](const double* w, double s, double z, int o, int c0) {
    uint32_t wd[3] = {0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const uint32_t q = (uint32_t)fmin(fmax(rint(w[j] / s) + z, 0.0), (double)qmax);
      const int b = bits * j;
      wd[b >> 5] |= q << (b & 31);
      if ((b & 31) + bits > 32) wd[(b >> 5) + 1] |= q >> (32 - (b & 31));
    }
    uint32_t* crow = codes + ((size_t)e * d_out + o) * wpr + (size_t)c0 * bits / 32;
    for (int t = 0; t < bits; ++t) crow[t] = wd[t];
  };
  if constexpr (LPG > 0) {
    const int nch = d_in >> 5;
    const size_t item = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool live = item < (size_t)d_out * nch;
    const int o = live ? (int)(item / nch) : 0;
    const int c = live ? (int)(item - (size_t)o * nch) : 0;
    double w[32];
    double mn = 0.0, mx = 0.0;
    if (live) {
      const size_t base = ((size_t)e * d_out + o) * d_in + (size_t)c * 32;
      const double* lrow = L + (size_t)o * d_in + (size_t)c * 32;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        w[j] = w_at<WDT>(W, base + j) - lrow[j];
        mn = fmin(mn, w[j]);
        mx = fmax(mx, w[j]);
      }
    }
#pragma unroll
    for (int off = LPG / 2; off > 0; off >>= 1) {
      mn = fmin(mn, __shfl_xor(mn, off, 64));
      mx = fmax(mx, __shfl_xor(mx, off, 64));
    }
    if (!live) return;
    double sv, zv;
    const int g = c / LPG;
    finish_scale(mn, mx, &sv, &zv, o, g);           // every lane of the group: the same values
    emit(w, sv, zv, o, c * 32);
  } else {
    const size_t item = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (item >= (size_t)d_out * ng) return;
    const int o = (int)(item / ng), g = (int)(item - (size_t)o * ng);
    const size_t wrow = ((size_t)e * d_out + o) * d_in + (size_t)g * G;
    const double* lrow = L + (size_t)o * d_in + (size_t)g * G;
    double mn = 0.0, mx = 0.0;
    for (int i = 0; i < G; ++i) {
      const double w = w_at<WDT>(W, wrow + i) - lrow[i];
      mn = fmin(mn, w);
      mx = fmax(mx, w);
    }
    double sv, zv;
    finish_scale(mn, mx, &sv, &zv, o, g);
    for (int c0 = 0; c0 < G; c0 += 32) {
      double w[32];
      for (int j = 0; j < 32; ++j) w[j] = w_at<WDT>(W, wrow + c0 + j) - lrow[c0 + j];
      emit(w, sv, zv, o, g * G + c0);
    }
  }
}

template <int WDT>
static void pk_rtn_w(const PackArgs& a, int e, const double* L, hipStream_t s) {
  const int lpg = a.group / 32;
  const size_t chunks = (size_t)a.d_out * (a.d_in / 32);
  const dim3 gc((unsigned)((chunks + 255) / 256));
#define PK_R(N) hipLaunchKernelGGL((pk_rtn_kernel<N, WDT>), gc, dim3(256), 0, s, a.W, e, a.d_out, \
                                   a.d_in, a.group, a.bits, L, a.codes, a.scales, a.zeros)
  switch (lpg) {
    case 1: PK_R(1); break;
    case 2: PK_R(2); break;
    case 4: PK_R(4); break;
    case 8: PK_R(8); break;
    case 16: PK_R(16); break;
    case 32: PK_R(32); break;
    case 64: PK_R(64); break;
    default: {
      const size_t items = (size_t)a.d_out * (a.d_in / a.group);
      hipLaunchKernelGGL((pk_rtn_kernel<0, WDT>), dim3((unsigned)((items + 255) / 256)), dim3(256), 0,
                         s, a.W, e, a.d_out, a.d_in, a.group, a.bits, L, a.codes, a.scales, a.zeros);
    }
  }
#undef PK_R
}

static void launch_pk_rtn(const PackArgs& a, int e, const double* L, hipStream_t s) {
  switch (a.wdt) {
    case 0: pk_rtn_w<0>(a, e, L, s); break;
    case 1: pk_rtn_w<1>(a, e, L, s); break;
    case 2: pk_rtn_w<2>(a, e, L, s); break;
    default: pk_rtn_w<3>(a, e, L, s); break;
  }
}

// ---- the pipeline ----------------------------------------------------------
struct PackPlan {
  size_t emap, Y, Q, Z, Gp, E, evec, eval, T, Sv, sig64, U64, V64, L, slabs, total;
  int gsplit;
};
constexpr int PK_WSPLIT = 4;     // split-K slabs of the W_big products

PackPlan pack_plan(int M, int N, int d_in, int d_out, int r, int l) {
  PackPlan p{};
  const size_t m = (size_t)M * d_out, n = (size_t)N * d_in;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = (o + bytes + 255) & ~(size_t)255;
    return at;
  };
  p.gsplit = (int)std::min<size_t>(64, std::max<size_t>(1, std::max(m, n) / 512));
  p.emap = take((size_t)M * N * 4);
  p.Y = take(m * l * 8);
  p.Q = take(m * l * 8);
  p.Z = take(n * l * 8);
  p.Gp = take((size_t)p.gsplit * l * l * 8);
  p.E = take((size_t)l * (l | 1) * 8);
  p.evec = take((size_t)l * l * 8);
  p.eval = take((size_t)l * 8);
  p.T = take((size_t)l * l * 8);
  p.Sv = take((size_t)l * std::max(r, 1) * 8);
  p.sig64 = take((size_t)std::max(r, 1) * 8);
  p.U64 = take(m * std::max(r, 1) * 8);
  p.V64 = take(n * std::max(r, 1) * 8);
  p.L = take((size_t)d_out * d_in * 8);
  p.slabs = take((size_t)PK_WSPLIT * std::max(m, n) * l * 8);
  p.total = o;
  return p;
}

template <typename X>
static X* at_ws(void* ws, size_t off) {
  return reinterpret_cast<X*>(reinterpret_cast<char*>(ws) + off);
}

// Gram matrix X^T X of X [rows][l] into split-K slabs, then its
// eigendecomposition and the whitening transform; Xo = X T.
static void orthonormalise(const double* X, size_t rows, int l, double* Xo, const PackPlan& p,
                           void* ws, hipStream_t s) {
  PkGemm g{};
  g.M = l;
  g.N = l;
  g.K = (int)rows;
  g.A = X;
  g.lda = l;
  g.B = X;
  g.ldb = l;
  g.C = at_ws<double>(ws, p.Gp);
  g.ldc = l;
  g.slab = (size_t)l * l;
  launch_pk_gemm(g, AM_DENSE_T, BM_DENSE, p.gsplit, s);
  const int nslab = pk_nslab((int)rows, p.gsplit);
  launch_pk_jacobi(at_ws<double>(ws, p.Gp), l, nslab, (size_t)l * l, at_ws<double>(ws, p.E),
                   at_ws<double>(ws, p.evec), at_ws<double>(ws, p.eval), 1e-24, s);
  hipLaunchKernelGGL(pk_whiten_kernel, dim3((l * l + 255) / 256), dim3(256), 0, s,
                     at_ws<double>(ws, p.evec), at_ws<double>(ws, p.eval), l, 1e-13,
                     at_ws<double>(ws, p.T));
  PkGemm h{};
  h.M = (int)rows;
  h.N = l;
  h.K = l;
  h.A = X;
  h.lda = l;
  h.B = at_ws<double>(ws, p.T);
  h.ldb = l;
  h.C = Xo;
  h.ldc = l;
  launch_pk_gemm(h, AM_DENSE, BM_DENSE, 1, s);
}

void run_pack(const PackArgs& a, void* ws, hipStream_t s) {
  const PackPlan p = pack_plan(a.M, a.N, a.d_in, a.d_out, a.rank, a.l);
  int* emap = at_ws<int>(ws, p.emap);
  (void)hipMemcpyAsync(emap, a.emap_host, sizeof(int) * a.M * a.N, hipMemcpyHostToDevice, s);
  const size_t m = (size_t)a.M * a.d_out, n = (size_t)a.N * a.d_in;
  const int l = a.l, r = a.rank;
  double* Y = at_ws<double>(ws, p.Y);
  double* Q = at_ws<double>(ws, p.Q);
  double* Z = at_ws<double>(ws, p.Z);
  PkGemm wb{};
  wb.W = a.W;
  wb.wdt = a.wdt;
  wb.d_out = a.d_out;
  wb.d_in = a.d_in;
  wb.Ng = a.N;
  wb.emap = emap;
  // Y = W_big Omega
  {
    PkGemm g = wb;
    g.M = (int)m;
    g.N = l;
    g.K = (int)n;
    g.B = a.omega;
    g.ldb = l;
    launch_pk_gemm_split(g, AM_WBIG, PK_WSPLIT, at_ws<double>(ws, p.slabs), Y, s);
  }
  orthonormalise(Y, m, l, Q, p, ws, s);
  orthonormalise(Q, m, l, Y, p, ws, s);      // second pass: the basis is in Y
  double* Qb = Y;
  double* Qs = Q;
  auto wt_times = [&](const double* X, double* out) {   // out [n][l] = W_big^T X
    PkGemm g = wb;
    g.M = (int)n;
    g.N = l;
    g.K = (int)m;
    g.B = X;
    g.ldb = l;
    launch_pk_gemm_split(g, AM_WBIG_T, PK_WSPLIT, at_ws<double>(ws, p.slabs), out, s);
  };
  for (int it = 0; it < a.power_iters; ++it) {
    wt_times(Qb, Z);
    PkGemm g = wb;                              // Y' = W_big Z
    g.M = (int)m;
    g.N = l;
    g.K = (int)n;
    g.B = Z;
    g.ldb = l;
    launch_pk_gemm_split(g, AM_WBIG, PK_WSPLIT, at_ws<double>(ws, p.slabs), Qs, s);
    orthonormalise(Qs, m, l, Qb, p, ws, s);
    orthonormalise(Qb, m, l, Qs, p, ws, s);
    std::swap(Qb, Qs);
  }
  // Z = W_big^T Q (= B^T); Z^T Z = B B^T
  wt_times(Qb, Z);
  {
    PkGemm g{};
    g.M = l;
    g.N = l;
    g.K = (int)n;
    g.A = Z;
    g.lda = l;
    g.B = Z;
    g.ldb = l;
    g.C = at_ws<double>(ws, p.Gp);
    g.ldc = l;
    g.slab = (size_t)l * l;
    launch_pk_gemm(g, AM_DENSE_T, BM_DENSE, p.gsplit, s);
    const int nslab = pk_nslab((int)n, p.gsplit);
    launch_pk_jacobi(at_ws<double>(ws, p.Gp), l, nslab, (size_t)l * l, at_ws<double>(ws, p.E),
                     at_ws<double>(ws, p.evec), at_ws<double>(ws, p.eval), 1e-24, s);
  }
  if (r > 0) {
    double* Sv = at_ws<double>(ws, p.Sv);
    double* sig64 = at_ws<double>(ws, p.sig64);
    hipLaunchKernelGGL(pk_vscale_kernel, dim3((l * r + 255) / 256), dim3(256), 0, s,
                       at_ws<double>(ws, p.evec), at_ws<double>(ws, p.eval), l, r, Sv, sig64);
    hipLaunchKernelGGL(pk_sigma_kernel, dim3(1), dim3(256), 0, s, sig64, r, a.sigma);
    // U = Q U~_r (into Z's space is not free: use U64 as the fp64 staging)
    double* U64 = at_ws<double>(ws, p.U64);
    double* V64 = at_ws<double>(ws, p.V64);
    {
      PkGemm g{};
      g.M = (int)m;
      g.N = r;
      g.K = l;
      g.A = Qb;
      g.lda = l;
      g.B = at_ws<double>(ws, p.evec);
      g.ldb = l;
      g.C = U64;
      g.ldc = r;
      launch_pk_gemm(g, AM_DENSE, BM_DENSE, 1, s);
      PkGemm h{};
      h.M = (int)n;
      h.N = r;
      h.K = l;
      h.A = Z;
      h.lda = l;
      h.B = Sv;
      h.ldb = r;
      h.C = V64;
      h.ldc = r;
      launch_pk_gemm(h, AM_DENSE, BM_DENSE, 1, s);
    }
    // stored factors, and their fp64 values (U times sigma32) in place
    const int bf = a.act_bf16;
    hipLaunchKernelGGL(pk_store_kernel, dim3((unsigned)std::min<size_t>((m * r + 255) / 256, 65536)),
                       dim3(256), 0, s, U64, (int)m, r, r, bf, reinterpret_cast<uint16_t*>(a.U),
                       a.sigma, U64);
    hipLaunchKernelGGL(pk_store_kernel, dim3((unsigned)std::min<size_t>((n * r + 255) / 256, 65536)),
                       dim3(256), 0, s, V64, (int)n, r, r, bf, reinterpret_cast<uint16_t*>(a.V),
                       nullptr, V64);
  }
  // per expert: L = block (m, n) of the stored low-rank product, then the
  // quantized residual
  double* Lb = at_ws<double>(ws, p.L);
  for (int e = 0; e < a.K; ++e) {
    const int mt = a.tile_host[e] / a.N, nt = a.tile_host[e] % a.N;
    if (r > 0) {
      PkGemm g{};
      g.M = a.d_out;
      g.N = a.d_in;
      g.K = r;
      g.A = at_ws<double>(ws, p.U64) + (size_t)mt * a.d_out * r;
      g.lda = r;
      g.B = at_ws<double>(ws, p.V64) + (size_t)nt * a.d_in * r;
      g.ldb = r;
      g.C = Lb;
      g.ldc = a.d_in;
      launch_pk_gemm(g, AM_DENSE, BM_DENSE_T, 1, s);
    } else {
      (void)hipMemsetAsync(Lb, 0, (size_t)a.d_out * a.d_in * 8, s);
    }
    launch_pk_rtn(a, e, Lb, s);
  }
}

size_t pack_workspace_bytes(int M, int N, int d_in, int d_out, int r, int l) {
  return pack_plan(M, N, d_in, d_out, r, l).total;
}

}  // namespace tq
