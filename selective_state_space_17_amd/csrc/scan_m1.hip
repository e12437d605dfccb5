// Mamba-1 selective scan forward for gfx950 (MI355X).
//
// The operation (per batch b, channel c, state n, time t):
//   h[n] <- exp(delta*A[c,n]) * h[n] + delta * B[b,t,n] * x[b,t,c]
//   out   = (sum_n C[b,t,n] h[n] + D[c] x) * silu(z)
// "03 - Modelos de espacio de estados": "El mecanismo selectivo de Mamba"
// (per-token B, C, delta), "Discretizacion" (zero-order hold, diagonal A so
// the exponential is elementwise), "Parallel scan" (the recurrence is
// associative, which is what lets the sequence be split below).
//
// Mapping onto the chip.  One wave (64 lanes) owns CPW = 64/G channels of
// one batch row and one time chunk; G lanes share a channel, each holding
// NPL of its states in fp32 VGPRs.  Per time tile of T steps the wave
// prefetches x/delta/z (and B/C, shared by all channels) with 16-byte
// global loads one tile ahead, stages them in its own LDS, then walks the
// tile step by step: per state one multiply for the exponent, one exp2
// (A is pre-scaled by log2 e), one multiply for delta*x*B, one FMA for the
// recurrence and one FMA for the readout.  The G partial readouts are summed
// with DPP row operations; outputs are staged in LDS and written back with
// 16-byte stores.  The kernels are VALU/transcendental bound (exp2 issues at
// half rate on gfx950), so everything else is kept off the VALU where it can
// be: B and C come from LDS as broadcast reads, the reduction rides on DPP.
//
// Sequence split (K > 1 chunks), exact up to fp32 rounding:
//   pass 1  every chunk scans from a zero state (chunk 0 from h0), writes its
//           outputs, its end state and the sum of its deltas S;
//   carry   per (b, c, n): h_in[k] = hend[k-1] + exp2(A' S[k-1]) h_in[k-1]
//           (the affine composition of consecutive chunks);
//   pass 2  chunks k >= 1 rescan from the true h_in[k], overwriting their
//           outputs, until the part of the state carried in from before the
//           chunk, bounded by exp2(max_n A'[n] * S_t) * max_n |h_in[n]|, is
//           below 2^-150 (it would round to zero in fp32); from there on the
//           pass-1 outputs are already correct.  A chunk holding a negative
//           delta, or a channel with A >= 0, is rescanned in full.
#include <type_traits>

#include "internal.h"

namespace mssm {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kWave = 64;

template <int IO> struct IoType;
template <> struct IoType<0> { using T = float; };
template <> struct IoType<1> { using T = uint16_t; };

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float v) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));   // v_cvt_pk_bf16_f32, round to nearest even
}

template <int CTRL> __device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Sum over each group of G consecutive lanes; every lane of the group gets the total.
template <int G> __device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  if constexpr (G >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  if constexpr (G >= 8) v += dpp<0x141>(v);   // row_half_mirror
  if constexpr (G >= 16) v += dpp<0x140>(v);  // row_mirror
  return v;
}

__device__ __forceinline__ float exp2_hw(float v) { return __builtin_amdgcn_exp2f(v); }

// modes
constexpr int kSingle = 0;   // whole sequence in one chunk: h0 -> final_state
constexpr int kChunk = 1;    // pass 1 of a split sequence
constexpr int kFixup = 2;    // pass 2 of a split sequence

template <int IO, int G, int NPL, bool VEC>
struct Geometry {
  using T = typename IoType<IO>::T;
  static constexpr int ES = sizeof(T);
  static constexpr int CPW = kWave / G;                          // channels per wave
  static constexpr int NP = G * NPL;                             // padded state count
  static constexpr int RB = CPW * ES;                            // bytes per tile row (one step)
  static constexpr int LPR = VEC ? (RB / 16 > 0 ? RB / 16 : 1) : 1;  // lanes per row for 16-byte loads
  static constexpr int RPI = VEC ? kWave / LPR : 1;              // rows per load instruction
  static constexpr int TG = G == 1 ? 16 : (G == 2 ? 32 : 64);
  static constexpr int TCAP = 4096 / NP < 8 ? 8 : 4096 / NP;     // keeps the fp32 B/C tiles <= 16 KB each
  static constexpr int STEPS = TG < TCAP ? TG : TCAP;            // steps per tile
  static constexpr bool VEC_OK = RB % 16 == 0 && kWave % LPR == 0 && STEPS % RPI == 0;
  static constexpr int NIT = VEC ? STEPS / RPI : (STEPS * CPW + kWave - 1) / kWave;  // x/delta/z loads per lane
  static constexpr int EPC = 16 / ES;                            // elements per 16-byte chunk
};

struct KernelParams {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* h0;
  void* out;
  float* final_state;
  float* hend;
  float* hin;
  float* S;
  int* neg;
  int64_t batch, L, dim, N;
  int64_t chunk_len;
  int K;
  int ngroups;          // channel groups (waves) per (batch, chunk)
  int chunk_offset;     // fix-up pass starts at chunk 1
};

template <int IO, int G, int NPL, bool VEC, int MODE>
__global__ __launch_bounds__(kWave) void scan_kernel(KernelParams p) {
  using Geo = Geometry<IO, G, NPL, VEC>;
  static_assert(!VEC || Geo::VEC_OK, "tile geometry");
  using T = typename Geo::T;
  constexpr int CPW = Geo::CPW, NP = Geo::NP, TT = Geo::STEPS, NIT = Geo::NIT;
  constexpr int EPC = Geo::EPC;
  // B/C tile: TT*N contiguous elements; 16-byte chunks when vectorised
  constexpr int BC_MAX_ELEMS = TT * NP;
  constexpr int NITB = VEC ? (BC_MAX_ELEMS * (int)sizeof(T) + 16 * kWave - 1) / (16 * kWave)
                           : (BC_MAX_ELEMS + kWave - 1) / kWave;

  __shared__ __attribute__((aligned(16))) T xs[TT * CPW];
  __shared__ __attribute__((aligned(16))) T ds[TT * CPW];
  __shared__ __attribute__((aligned(16))) T zs[TT * CPW];
  __shared__ __attribute__((aligned(16))) T ys[TT * CPW];
  __shared__ __attribute__((aligned(16))) float Bs[TT * NP];
  __shared__ __attribute__((aligned(16))) float Cs[TT * NP];

  const int lane = threadIdx.x;
  const int ch = lane / G;
  const int g = lane % G;

  // block -> (batch, chunk, channel group)
  int bid = blockIdx.x;
  const int cg = bid % p.ngroups;
  bid /= p.ngroups;
  const int nchunks_here = (MODE == kFixup) ? p.K - 1 : p.K;
  const int k = bid % nchunks_here + p.chunk_offset;
  const int64_t b = bid / nchunks_here;

  const int64_t dim = p.dim, N = p.N, L = p.L;
  const int64_t c0 = static_cast<int64_t>(cg) * CPW;
  const int64_t c = c0 + ch;
  const bool cvalid = c < dim;
  const int64_t t_begin = static_cast<int64_t>(k) * p.chunk_len;
  const int64_t t_end = t_begin + p.chunk_len < L ? t_begin + p.chunk_len : L;

  const T* __restrict__ xg = static_cast<const T*>(p.x);
  const T* __restrict__ dg = static_cast<const T*>(p.delta);
  const T* __restrict__ zg = static_cast<const T*>(p.z);
  const T* __restrict__ Bg = static_cast<const T*>(p.B);
  const T* __restrict__ Cg = static_cast<const T*>(p.C);
  T* __restrict__ yg = static_cast<T*>(p.out);
  const bool has_z = p.z != nullptr;

  // per-lane constants and state
  float A2[NPL], h[NPL];
  float amax = -INFINITY;     // largest (least negative) exponent slope among real states
  float hmax = 0.f;           // largest |h_in| among real states (fix-up)
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int64_t n = static_cast<int64_t>(g) * NPL + j;
    const bool real = cvalid && n < N;
    A2[j] = real ? p.A[c * N + n] * kLog2e : 0.f;
    float h_init = 0.f;
    if constexpr (MODE == kFixup) {
      h_init = real ? p.hin[((b * p.K + k) * dim + c) * N + n] : 0.f;
    } else {
      if (p.h0 != nullptr && real && (MODE == kSingle || k == 0)) h_init = p.h0[(b * dim + c) * N + n];
    }
    h[j] = h_init;
    if (real) {
      amax = fmaxf(amax, A2[j]);
      hmax = fmaxf(hmax, fabsf(h_init));
    }
  }
  const float Dc = (p.D != nullptr && cvalid) ? p.D[c] : 0.f;

  bool fix_done = false;
  bool never_exit = false;
  if constexpr (MODE == kFixup) {
    // a channel whose chunk saw a negative delta cannot use the decay bound
    never_exit = cvalid && p.neg[(b * p.K + k) * dim + c] != 0;
  }
  float S = 0.f;       // running sum of delta over this chunk
  int negseen = 0;

  // zero the padded B/C columns once (never overwritten by loads)
  if (NP > N) {
    for (int e = lane; e < TT * NP; e += kWave) {
      if ((e % NP) >= N) { Bs[e] = 0.f; Cs[e] = 0.f; }
    }
  }

  // ------------------------------------------------------------------
  // prefetch registers
  // ------------------------------------------------------------------
  using Chunk = typename std::conditional<VEC, uint4, T>::type;
  Chunk xr[NIT], dr[NIT], zr[NIT];
  Chunk br[NITB], cr[NITB];

  auto issue_loads = [&](int64_t t0) {
    const int64_t nvalid = (t_end - t0) < TT ? (t_end - t0) : TT;
    if constexpr (VEC) {
      const int rin = lane / Geo::LPR, seg = lane % Geo::LPR;
      const int64_t cc = c0 + static_cast<int64_t>(seg) * EPC;
#pragma unroll
      for (int i = 0; i < NIT; ++i) {
        const int r = i * Geo::RPI + rin;
        const bool ok = r < nvalid && cc < dim;
        const int64_t off = ((b * L + t0 + r) * dim + cc);
        xr[i] = ok ? *reinterpret_cast<const uint4*>(xg + off) : uint4{0, 0, 0, 0};
        dr[i] = ok ? *reinterpret_cast<const uint4*>(dg + off) : uint4{0, 0, 0, 0};
        if (has_z) zr[i] = ok ? *reinterpret_cast<const uint4*>(zg + off) : uint4{0, 0, 0, 0};
      }
      const int64_t nbc = nvalid * N;    // valid elements of the flattened [steps x N] B/C tile
      const int64_t base = (b * L + t0) * N;
#pragma unroll
      for (int i = 0; i < NITB; ++i) {
        const int64_t e = (static_cast<int64_t>(i) * kWave + lane) * EPC;
        const bool ok = e < nbc;
        br[i] = ok ? *reinterpret_cast<const uint4*>(Bg + base + e) : uint4{0, 0, 0, 0};
        cr[i] = ok ? *reinterpret_cast<const uint4*>(Cg + base + e) : uint4{0, 0, 0, 0};
      }
    } else {
#pragma unroll
      for (int i = 0; i < NIT; ++i) {
        const int e = i * kWave + lane;
        const int r = e / CPW, col = e % CPW;
        const bool ok = e < TT * CPW && r < nvalid && c0 + col < dim;
        const int64_t off = (b * L + t0 + r) * dim + c0 + col;
        xr[i] = ok ? xg[off] : T(0);
        dr[i] = ok ? dg[off] : T(0);
        if (has_z) zr[i] = ok ? zg[off] : T(0);
      }
      const int64_t nbc = nvalid * N;
      const int64_t base = (b * L + t0) * N;
#pragma unroll
      for (int i = 0; i < NITB; ++i) {
        const int64_t e = static_cast<int64_t>(i) * kWave + lane;
        const bool ok = e < nbc;
        br[i] = ok ? Bg[base + e] : T(0);
        cr[i] = ok ? Cg[base + e] : T(0);
      }
    }
  };

  auto stage_to_lds = [&](int64_t t0) {
    const int64_t nvalid = (t_end - t0) < TT ? (t_end - t0) : TT;
    if constexpr (VEC) {
      const int rin = lane / Geo::LPR, seg = lane % Geo::LPR;
#pragma unroll
      for (int i = 0; i < NIT; ++i) {
        const int r = i * Geo::RPI + rin;
        const int idx = r * CPW + seg * EPC;
        *reinterpret_cast<uint4*>(&xs[idx]) = xr[i];
        *reinterpret_cast<uint4*>(&ds[idx]) = dr[i];
        if (has_z) *reinterpret_cast<uint4*>(&zs[idx]) = zr[i];
      }
      const int64_t nbc = nvalid * N;
#pragma unroll
      for (int i = 0; i < NITB; ++i) {
        const int64_t e = (static_cast<int64_t>(i) * kWave + lane) * EPC;
        if (e < nbc) {
          const T* bv = reinterpret_cast<const T*>(&br[i]);
          const T* cv = reinterpret_cast<const T*>(&cr[i]);
#pragma unroll
          for (int q = 0; q < EPC; ++q) {
            const int64_t ee = e + q;
            const int r = static_cast<int>(ee / N), n = static_cast<int>(ee % N);
            Bs[r * NP + n] = to_f32(bv[q]);
            Cs[r * NP + n] = to_f32(cv[q]);
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NIT; ++i) {
        const int e = i * kWave + lane;
        if (e < TT * CPW) {
          xs[e] = xr[i];
          ds[e] = dr[i];
          if (has_z) zs[e] = zr[i];
        }
      }
      const int64_t nbc = nvalid * N;
#pragma unroll
      for (int i = 0; i < NITB; ++i) {
        const int64_t e = static_cast<int64_t>(i) * kWave + lane;
        if (e < nbc) {
          const int r = static_cast<int>(e / N), n = static_cast<int>(e % N);
          Bs[r * NP + n] = to_f32(br[i]);
          Cs[r * NP + n] = to_f32(cr[i]);
        }
      }
    }
  };

  auto store_tile = [&](int64_t t0) {
    const int64_t nvalid = (t_end - t0) < TT ? (t_end - t0) : TT;
    if constexpr (VEC) {
      const int rin = lane / Geo::LPR, seg = lane % Geo::LPR;
      const int64_t cc = c0 + static_cast<int64_t>(seg) * EPC;
#pragma unroll
      for (int i = 0; i < NIT; ++i) {
        const int r = i * Geo::RPI + rin;
        if (r < nvalid && cc < dim) {
          const uint4 v = *reinterpret_cast<const uint4*>(&ys[r * CPW + seg * EPC]);
          *reinterpret_cast<uint4*>(yg + (b * L + t0 + r) * dim + cc) = v;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NIT; ++i) {
        const int e = i * kWave + lane;
        const int r = e / CPW, col = e % CPW;
        if (e < TT * CPW && r < nvalid && c0 + col < dim) yg[(b * L + t0 + r) * dim + c0 + col] = ys[e];
      }
    }
  };

  // ------------------------------------------------------------------
  // time loop
  // ------------------------------------------------------------------
  if (t_begin < t_end) issue_loads(t_begin);
  int64_t prev_t0 = -1;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += TT) {
    const int ns = (t_end - t0) < TT ? static_cast<int>(t_end - t0) : TT;
    stage_to_lds(t0);
    __syncthreads();
    if (prev_t0 >= 0) store_tile(prev_t0);
    if (t0 + TT < t_end) issue_loads(t0 + TT);

    for (int s = 0; s < ns; ++s) {
      const float d = to_f32(ds[s * CPW + ch]);
      const float u = to_f32(xs[s * CPW + ch]);
      const float du = d * u;
      const float4* bp = reinterpret_cast<const float4*>(&Bs[s * NP + g * NPL]);
      const float4* cp = reinterpret_cast<const float4*>(&Cs[s * NP + g * NPL]);
      float acc = 0.f;
#pragma unroll
      for (int q = 0; q < NPL / 4; ++q) {
        const float4 bq = bp[q];
        const float4 cq = cp[q];
        const float bb[4] = {bq.x, bq.y, bq.z, bq.w};
        const float cc4[4] = {cq.x, cq.y, cq.z, cq.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = q * 4 + r;
          const float dA = exp2_hw(d * A2[j]);
          h[j] = __builtin_fmaf(dA, h[j], du * bb[r]);
          acc = __builtin_fmaf(cc4[r], h[j], acc);
        }
      }
      acc = group_sum<G>(acc);
      float y = __builtin_fmaf(Dc, u, acc);
      if (has_z) {
        const float zz = to_f32(zs[s * CPW + ch]);
        y *= zz * __builtin_amdgcn_rcpf(1.f + exp2_hw(-zz * kLog2e));
      }
      ys[s * CPW + ch] = from_f32<T>(y);
      if constexpr (MODE != kSingle) {
        S += d;
        negseen |= (d < 0.f);
      }
    }
    __syncthreads();
    prev_t0 = t0;

    if constexpr (MODE == kFixup) {
      // carried-in part bounded by exp2(amax * S) * hmax; done once it would be 0 in fp32
      const bool lane_done = !cvalid || hmax == 0.f ||
                             (!never_exit && amax < 0.f && amax * S + __log2f(hmax) < -150.f);
      if (__all(lane_done)) {
        fix_done = true;
        break;
      }
    }
  }
  if (prev_t0 >= 0) store_tile(prev_t0);
  (void)fix_done;

  // ------------------------------------------------------------------
  // chunk results
  // ------------------------------------------------------------------
  if constexpr (MODE == kSingle) {
    if (p.final_state != nullptr && cvalid) {
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        const int64_t n = static_cast<int64_t>(g) * NPL + j;
        if (n < N) p.final_state[(b * dim + c) * N + n] = h[j];
      }
    }
  } else if constexpr (MODE == kChunk) {
    if (cvalid) {
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        const int64_t n = static_cast<int64_t>(g) * NPL + j;
        if (n < N) p.hend[((b * p.K + k) * dim + c) * N + n] = h[j];
      }
      if (g == 0) {
        p.S[(b * p.K + k) * dim + c] = S;
        p.neg[(b * p.K + k) * dim + c] = negseen;
      }
    }
  }
}

// carry across chunks: one thread per (b, c, n)
__global__ __launch_bounds__(256) void carry_kernel(KernelParams p) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = p.batch * p.dim * p.N;
  if (idx >= total) return;
  const int64_t n = idx % p.N;
  const int64_t c = (idx / p.N) % p.dim;
  const int64_t b = idx / (p.N * p.dim);
  const float a2 = p.A[c * p.N + n] * kLog2e;
  float h = p.hend[((b * p.K + 0) * p.dim + c) * p.N + n];
  for (int k = 1; k < p.K; ++k) {
    p.hin[((b * p.K + k) * p.dim + c) * p.N + n] = h;
    const float s = p.S[(b * p.K + k) * p.dim + c];
    h = __builtin_fmaf(exp2_hw(a2 * s), h, p.hend[((b * p.K + k) * p.dim + c) * p.N + n]);
  }
  if (p.final_state != nullptr) p.final_state[(b * p.dim + c) * p.N + n] = h;
}

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

template <int IO, int G, int NPL, bool VEC>
hipError_t launch_cfg(const KernelParams& kp, int64_t batch, hipStream_t stream) {
  const dim3 block(kWave);
  if (kp.K == 1) {
    const dim3 grid(static_cast<unsigned>(batch * kp.ngroups));
    hipLaunchKernelGGL((scan_kernel<IO, G, NPL, VEC, kSingle>), grid, block, 0, stream, kp);
    return hipGetLastError();
  }
  {
    const dim3 grid(static_cast<unsigned>(batch * kp.K * kp.ngroups));
    hipLaunchKernelGGL((scan_kernel<IO, G, NPL, VEC, kChunk>), grid, block, 0, stream, kp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int64_t total = batch * kp.dim * kp.N;
    const dim3 grid(static_cast<unsigned>((total + 255) / 256));
    hipLaunchKernelGGL(carry_kernel, grid, dim3(256), 0, stream, kp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    KernelParams kf = kp;
    kf.chunk_offset = 1;
    const dim3 grid(static_cast<unsigned>(batch * (kp.K - 1) * kp.ngroups));
    hipLaunchKernelGGL((scan_kernel<IO, G, NPL, VEC, kFixup>), grid, block, 0, stream, kf);
    return hipGetLastError();
  }
}

template <int IO, int G, int NPL>
hipError_t launch_vec(const KernelParams& kp, bool vec, int64_t batch, hipStream_t stream) {
  if constexpr (Geometry<IO, G, NPL, true>::VEC_OK) {
    if (vec) return launch_cfg<IO, G, NPL, true>(kp, batch, stream);
  }
  return launch_cfg<IO, G, NPL, false>(kp, batch, stream);
}

template <int IO, int G>
hipError_t launch_npl(const KernelParams& kp, int npl, bool vec, int64_t batch, hipStream_t stream) {
  switch (npl) {
    case 4: return launch_vec<IO, G, 4>(kp, vec, batch, stream);
    case 8: return launch_vec<IO, G, 8>(kp, vec, batch, stream);
    default: return launch_vec<IO, G, 16>(kp, vec, batch, stream);
  }
}

template <int IO>
hipError_t launch_io(const KernelParams& kp, int G, int npl, bool vec, int64_t batch, hipStream_t stream) {
  switch (G) {
    case 1: return launch_npl<IO, 1>(kp, npl, vec, batch, stream);
    case 2: return launch_npl<IO, 2>(kp, npl, vec, batch, stream);
    case 4: return launch_npl<IO, 4>(kp, npl, vec, batch, stream);
    case 8: return launch_npl<IO, 8>(kp, npl, vec, batch, stream);
    default: return launch_npl<IO, 16>(kp, npl, vec, batch, stream);
  }
}

int states_per_lane(int G, int64_t N) {
  const int64_t need = (N + G - 1) / G;
  return need <= 4 ? 4 : (need <= 8 ? 8 : 16);
}

}  // namespace

bool scan_supported_G(int G, int64_t N) {
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return false;
  return static_cast<int64_t>(G) * 16 >= N;
}

size_t scan_workspace_bytes(int64_t batch, int64_t dim, int64_t N, int K) {
  if (K <= 1) return 0;
  const size_t st = static_cast<size_t>(batch) * K * dim * N * sizeof(float);
  const size_t sc = static_cast<size_t>(batch) * K * dim * sizeof(float);
  return 2 * align256(st) + 2 * align256(sc);
}

hipError_t scan_launch(const ScanArgs& a, hipStream_t stream) {
  KernelParams kp{};
  kp.x = a.x; kp.delta = a.delta; kp.A = a.A; kp.B = a.B; kp.C = a.C; kp.D = a.D; kp.z = a.z; kp.h0 = a.h0;
  kp.out = a.out; kp.final_state = a.final_state;
  kp.batch = a.batch; kp.L = a.L; kp.dim = a.dim; kp.N = a.N;
  kp.K = a.K;
  kp.chunk_len = (a.L + a.K - 1) / a.K;
  kp.chunk_offset = 0;
  const int G = a.G;
  const int cpw = kWave / G;
  kp.ngroups = static_cast<int>((a.dim + cpw - 1) / cpw);
  if (a.K > 1) {
    char* ws = static_cast<char*>(a.workspace);
    const size_t st = static_cast<size_t>(a.batch) * a.K * a.dim * a.N * sizeof(float);
    const size_t sc = static_cast<size_t>(a.batch) * a.K * a.dim * sizeof(float);
    kp.hend = reinterpret_cast<float*>(ws);
    kp.hin = reinterpret_cast<float*>(ws + align256(st));
    kp.S = reinterpret_cast<float*>(ws + 2 * align256(st));
    kp.neg = reinterpret_cast<int*>(ws + 2 * align256(st) + align256(sc));
  }
  const int npl = states_per_lane(G, a.N);
  const size_t es = a.io == 1 ? 2 : 4;
  auto al16 = [](const void* q) { return q == nullptr || (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  const bool vec = (a.dim * es) % 16 == 0 && (a.N * es) % 16 == 0 && al16(a.x) && al16(a.delta) && al16(a.z) &&
                   al16(a.B) && al16(a.C) && al16(a.out);
  if (a.io == 1) return launch_io<1>(kp, G, npl, vec, a.batch, stream);
  return launch_io<0>(kp, G, npl, vec, a.batch, stream);
}

}  // namespace mssm
