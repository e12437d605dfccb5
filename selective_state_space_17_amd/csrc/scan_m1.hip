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
// Mapping onto the chip.  A block of 4 waves owns CPB = 256/G channels of one
// batch row and one time chunk; G lanes share a channel, each holding NPL of
// its states in fp32 VGPRs.  The path is VALU/transcendental bound (exp2
// issues at half rate on gfx950), so per state update the lane issues only
// the five unavoidable operations: a multiply for the exponent (A is
// pre-scaled by log2 e), exp2, a multiply for delta*x*B, an FMA for the
// recurrence and an FMA for the readout.  Everything per (t, c) -- bf16
// widening, delta*x, the silu gate, D*x -- is computed once per element when a
// time tile is staged (global -> registers one tile ahead with 16-byte loads,
// then into fp32 LDS arrays), not once per lane; outputs are collected in LDS
// and written back with 16-byte stores.
//
// B and C (shared by all channels of a batch row) reach the lanes in two ways:
//  - dstate <= 16 ("fast" path): one VGPR per step holds the 16 values across
//    each 16-lane row and every state reads its value through a DPP operand
//    (row_newbcast for one lane per channel, quad_perm broadcasts for 2 or 4
//    lanes per channel; the lane layout puts a state group on one quad), so
//    B rides on v_mul_f32_dpp and C on v_fmac_f32_dpp at no extra cost;
//  - larger dstate ("generic" path): per-lane 16-byte LDS reads.
// The G partial readouts are summed with DPP row rotations/permutations.
//
// Sequence split (K > 1 chunks), exact up to fp32 rounding:
//   pass 1  every chunk scans from a zero state (chunk 0 from h0), writes its
//           outputs, its end state and the sum of its deltas S;
//   carry   per (b, c, n): h_in[k] = hend[k-1] + exp2(A' S[k-1]) h_in[k-1]
//           (the affine composition of consecutive chunks), taken as a
//           wave-level parallel scan over the chunks' maps;
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
constexpr int kWaves = 4;      // waves per block
constexpr int kThreads = kWave * kWaves;

using u32x4 = unsigned int __attribute__((ext_vector_type(4)));   // native 128-bit register tuple

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
// the same with bound_ctrl set, for controls whose every source lane exists (a row rotation): the
// compiler then folds the move into the consuming VALU op
template <int CTRL> __device__ __forceinline__ float dpp_bc(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}

__device__ __forceinline__ float exp2_hw(float v) { return __builtin_amdgcn_exp2f(v); }

__device__ __forceinline__ float silu_gate(float z) {
  return z * __builtin_amdgcn_rcpf(1.f + exp2_hw(-z * kLog2e));
}

// modes
constexpr int kSingle = 0;   // whole sequence in one chunk: h0 -> final_state
constexpr int kChunk = 1;    // pass 1 of a split sequence
constexpr int kFixup = 2;    // pass 2 of a split sequence

// DPP controls
constexpr int kRowRor8 = 0x128;
constexpr int kRowRor4 = 0x124;
constexpr int kQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
constexpr int quad_bcast(int j) { return j | (j << 2) | (j << 4) | (j << 6); }   // quad_perm [j,j,j,j]
constexpr int row_newbcast(int j) { return 0x150 + j; }

template <int IO, int G, int NPL, bool VEC, bool FAST>
struct Geometry {
  using T = typename IoType<IO>::T;
  static constexpr int ES = sizeof(T);
  static constexpr int CPW = kWave / G;                          // channels per wave
  static constexpr int CPB = kWaves * CPW;                       // channels per block
  static constexpr int NP = FAST ? 16 : G * NPL;                 // padded state count
  static constexpr int RB = CPB * ES;                            // bytes per tile row (one step)
  static constexpr int LPR = VEC ? (RB / 16 > 0 ? RB / 16 : 1) : 1;  // threads per row for 16-byte loads
  static constexpr int RPI = VEC ? (kThreads / LPR > 0 ? kThreads / LPR : 1) : 1;  // rows per load instruction
  static constexpr int TWANT = 4096 / CPB < 32 ? 4096 / CPB : 32;  // <= 32 unrolled steps, operand tiles <= 64 KB
  static constexpr int TCAP = 4096 / NP < 8 ? 8 : 4096 / NP;    // B/C tiles stay <= 16 KB each
  static constexpr int STEPS = TWANT < TCAP ? TWANT : TCAP;      // steps per tile
  static constexpr bool VEC_OK = RB % 16 == 0 && kThreads % LPR == 0 && STEPS % RPI == 0;
  static constexpr int NIT = VEC ? STEPS / RPI : (STEPS * CPB + kThreads - 1) / kThreads;  // loads per thread
  static constexpr int EPC = 16 / ES;                            // elements per 16-byte chunk
  static constexpr int EPT = VEC ? EPC : 1;                      // channels a staging thread holds
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
  int ngroups;          // channel groups (blocks) per (batch, chunk)
  int chunk_offset;     // fix-up pass starts at chunk 1
  int bc_shift;         // log2(N / elements-per-16-bytes) for 16-byte B/C loads
  // short causal convolution in front of the scan (wide kernel, CONV = true):
  // x above is then the convolution's input
  const float* conv_w;     // [dim, conv_width]
  const float* conv_b;     // [dim], nullable
  const void* conv_init;   // [batch, conv_width - 1, dim] (io dtype), nullable
  int conv_width;          // 1..4
  // training mode (wide kernel): the state entering every 16-step tile,
  // [batch][ckpt_tiles][16 * ngroups][16] fp32, for the gradient kernel
  float* ckpt;
  int64_t ckpt_tiles;
};

// Readout for the fast path: a0 + a1 = sum_j C_j * h_j with C_j taken from the
// lane holding it through a DPP operand (v_mul/v_fmac_f32_dpp); two partial
// sums keep the dependent chain short.  s_nop 1 covers the VALU-write ->
// DPP-read hazard on the C register.
template <int G> struct FastReadout;

template <> struct FastReadout<1> {   // one VGPR, C[n] in lane n of each row: row_newbcast:n
  static __device__ __forceinline__ void run(float& a0, float& a1, float c, const float (&h)[16]) {
    asm("s_nop 1\n\t"
        "v_mul_f32_dpp %0, %2, %3 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %2, %4 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %5 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %2, %6 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %7 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %2, %8 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %9 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %2, %10 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %11 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %2, %12 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %13 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %2, %14 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %15 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %2, %16 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %17 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %2, %18 row_newbcast:15 row_mask:0xf bank_mask:0xf"
        : "=&v"(a0), "=&v"(a1)
        : "v"(c), "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]), "v"(h[4]), "v"(h[5]), "v"(h[6]), "v"(h[7]),
          "v"(h[8]), "v"(h[9]), "v"(h[10]), "v"(h[11]), "v"(h[12]), "v"(h[13]), "v"(h[14]), "v"(h[15]));
  }
};

template <> struct FastReadout<2> {   // two VGPRs, quad position p holds C[8g + 4v + p]: quad_perm [p,p,p,p]
  static __device__ __forceinline__ void run(float& a0, float& a1, float c0, float c1, const float (&h)[8]) {
    asm("s_nop 1\n\t"
        "v_mul_f32_dpp %0, %2, %4 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %2, %5 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %6 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %2, %7 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %3, %8 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %3, %9 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %3, %10 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %3, %11 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf"
        : "=&v"(a0), "=&v"(a1)
        : "v"(c0), "v"(c1), "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]), "v"(h[4]), "v"(h[5]), "v"(h[6]),
          "v"(h[7]));
  }
};

template <> struct FastReadout<4> {   // one VGPR, quad position p holds C[4g + p]
  static __device__ __forceinline__ void run(float& a0, float& a1, float c, const float (&h)[4]) {
    asm("s_nop 1\n\t"
        "v_mul_f32_dpp %0, %2, %3 quad_perm:[0,0,0,0] row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %2, %4 quad_perm:[1,1,1,1] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %5 quad_perm:[2,2,2,2] row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %2, %6 quad_perm:[3,3,3,3] row_mask:0xf bank_mask:0xf"
        : "=&v"(a0), "=&v"(a1)
        : "v"(c), "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]));
  }
};

// B_j for state j of the lane's state group, through a DPP operand
template <int G, int J> __device__ __forceinline__ float fast_b(float b0, float b1) {
  if constexpr (G == 1) return dpp<row_newbcast(J)>(b0);
  else if constexpr (G == 2) return J < 4 ? dpp<quad_bcast(J & 3)>(b0) : dpp<quad_bcast(J & 3)>(b1);
  else return dpp<quad_bcast(J)>(b0);
}

template <int G, int J, int NPL>
__device__ __forceinline__ void fast_updates(float (&h)[NPL], const float (&A2)[NPL], float d, float du, float b0,
                                             float b1) {
  const float dA = exp2_hw(d * A2[J]);
  h[J] = __builtin_fmaf(dA, h[J], du * fast_b<G, J>(b0, b1));
  if constexpr (J + 1 < NPL) fast_updates<G, J + 1, NPL>(h, A2, d, du, b0, b1);
}

// Sum of the G partial readouts of a channel (every lane of the group gets it).
template <int G, bool FAST> __device__ __forceinline__ float reduce_groups(float v) {
  if constexpr (FAST) {
    // state groups sit on different quads (G=4) or quad pairs (G=2) of a row
    if constexpr (G >= 2) v += dpp<kRowRor8>(v);
    if constexpr (G >= 4) v += dpp<kRowRor4>(v);
  } else {
    // generic layout: the G lanes of a channel are consecutive
    if constexpr (G >= 2) v += dpp<kQuadSwap1>(v);
    if constexpr (G >= 4) v += dpp<kQuadSwap2>(v);
    if constexpr (G >= 8) v += dpp<kRowHalfMirror>(v);
    if constexpr (G >= 16) v += dpp<kRowMirror>(v);
  }
  return v;
}

template <int IO, int G, int NPL, bool VEC, bool FAST, int MODE>
__global__ __launch_bounds__(kThreads) void scan_kernel(KernelParams p) {
  using Geo = Geometry<IO, G, NPL, VEC, FAST>;
  static_assert(!VEC || Geo::VEC_OK, "tile geometry");
  static_assert(!FAST || (G * NPL == 16 && (G == 1 || G == 2 || G == 4)), "fast path layout");
  using T = typename Geo::T;
  constexpr int CPW = Geo::CPW, CPB = Geo::CPB, NP = Geo::NP, TT = Geo::STEPS, NIT = Geo::NIT;
  constexpr int EPC = Geo::EPC, EPT = Geo::EPT;
  constexpr int NITB = VEC ? (TT * NP * static_cast<int>(sizeof(T)) + 16 * kThreads - 1) / (16 * kThreads)
                           : (TT * NP + kThreads - 1) / kThreads;

  // per-(t, c) operands, fp32, with one spare row so a step can always read one ahead
  __shared__ __attribute__((aligned(16))) float Dl[(TT + 1) * CPB];   // delta
  __shared__ __attribute__((aligned(16))) float Ul[(TT + 1) * CPB];   // delta * x
  __shared__ __attribute__((aligned(16))) float Gl[(TT + 1) * CPB];   // silu(z) (1 without z)
  __shared__ __attribute__((aligned(16))) float Yl[(TT + 1) * CPB];   // silu(z) * D * x
  __shared__ __attribute__((aligned(16))) T ys[TT * CPB];            // outputs of the previous tile
  __shared__ __attribute__((aligned(16))) float Bs[(TT + 1) * NP];
  __shared__ __attribute__((aligned(16))) float Cs[(TT + 1) * NP];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  // lane -> (channel within the wave, state group)
  int chw, g;
  if constexpr (FAST && G == 2) {
    const int r = lane >> 4, q = (lane >> 2) & 3, pp = lane & 3;
    g = q >> 1;
    chw = 8 * r + 4 * (q & 1) + pp;
  } else if constexpr (FAST && G == 4) {
    g = (lane >> 2) & 3;
    chw = 4 * (lane >> 4) + (lane & 3);
  } else {
    chw = lane / G;
    g = lane % G;
  }
  const int chb = wave * CPW + chw;   // channel within the block

  // block -> (batch, chunk, channel group)
  int bid = blockIdx.x;
  const int cg = bid % p.ngroups;
  bid /= p.ngroups;
  const int nchunks_here = (MODE == kFixup) ? p.K - 1 : p.K;
  const int k = bid % nchunks_here + p.chunk_offset;
  const int64_t b = bid / nchunks_here;

  const int64_t dim = p.dim, N = p.N, L = p.L;
  const int64_t c0 = static_cast<int64_t>(cg) * CPB;
  const int64_t c = c0 + chb;
  const bool cvalid = c < dim;
  const int64_t t_begin = static_cast<int64_t>(k) * p.chunk_len;
  const int64_t t_end = t_begin + p.chunk_len < L ? t_begin + p.chunk_len : L;

  const T* __restrict__ xg = static_cast<const T*>(p.x);
  const T* __restrict__ dg = static_cast<const T*>(p.delta);
  // without z the z loads read x (values unused) so the load stream has no branches
  const T* __restrict__ zg = static_cast<const T*>(p.z != nullptr ? p.z : p.x);
  const T* __restrict__ Bg = static_cast<const T*>(p.B);
  const T* __restrict__ Cg = static_cast<const T*>(p.C);
  T* __restrict__ yg = static_cast<T*>(p.out);
  const bool has_z = p.z != nullptr;
  const int Ni = static_cast<int>(N);

  // states of this lane: n = g*NPL + j
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

  bool never_exit = false;
  if constexpr (MODE == kFixup) {
    // a channel whose chunk saw a negative delta cannot use the decay bound
    never_exit = cvalid && p.neg[(b * p.K + k) * dim + c] != 0;
  }
  float S = 0.f;       // running sum of delta over this chunk
  int negseen = 0;

  // staging threads: the channels they widen are fixed for the whole kernel
  const int rin = VEC ? tid / Geo::LPR : 0;
  const int seg = VEC ? tid % Geo::LPR : 0;
  const int scol = VEC ? seg * EPC : tid % CPB;    // first channel (within block) of this thread
  float Dreg[EPT];
#pragma unroll
  for (int q = 0; q < EPT; ++q) {
    const int64_t cc = c0 + scol + q;
    Dreg[q] = (p.D != nullptr && cc < dim) ? p.D[cc] : 0.f;
  }

  // zero the padded B/C columns and the spare rows once (loads never write them)
  for (int e = tid; e < (TT + 1) * NP; e += kThreads) {
    if ((e % NP) >= Ni || e >= TT * NP) {
      Bs[e] = 0.f;
      Cs[e] = 0.f;
    }
  }
  for (int e = tid; e < CPB; e += kThreads) {
    Dl[TT * CPB + e] = 0.f;
    Ul[TT * CPB + e] = 0.f;
    Gl[TT * CPB + e] = 0.f;
    Yl[TT * CPB + e] = 0.f;
  }

  // ------------------------------------------------------------------
  // tile prefetch registers, filled one (long) tile ahead of use
  // ------------------------------------------------------------------
  using Chunk = typename std::conditional<VEC, u32x4, T>::type;
  Chunk xr[NIT], dr[NIT], zr[NIT];
  Chunk br[NITB], cr[NITB];

  // Loads are unconditional: out-of-range rows/channels/chunks are clamped to
  // in-range addresses; their values land in LDS rows or channels that are
  // never used.
  auto issue_loads = [&](int64_t t0) {
    const int nvalid = static_cast<int>((t_end - t0) < TT ? (t_end - t0) : TT);
    if constexpr (VEC) {
      const int64_t cc = (c0 + scol) < dim ? (c0 + scol) : (dim - EPC);
#pragma unroll
      for (int i = 0; i < NIT; ++i) {
        const int r = i * Geo::RPI + rin;
        const int rr = r < nvalid ? r : nvalid - 1;
        const int64_t off = (b * L + t0 + rr) * dim + cc;
        xr[i] = *reinterpret_cast<const u32x4*>(xg + off);
        dr[i] = *reinterpret_cast<const u32x4*>(dg + off);
        zr[i] = *reinterpret_cast<const u32x4*>(zg + off);
      }
      // the [steps x N] B/C tile is contiguous in memory: 16-byte chunks
      const int nchunks = (nvalid * Ni) / EPC;
      const int64_t base = (b * L + t0) * N;
#pragma unroll
      for (int i = 0; i < NITB; ++i) {
        const int ci = i * kThreads + tid;
        const int cci = ci < nchunks ? ci : nchunks - 1;
        br[i] = *reinterpret_cast<const u32x4*>(Bg + base + static_cast<int64_t>(cci) * EPC);
        cr[i] = *reinterpret_cast<const u32x4*>(Cg + base + static_cast<int64_t>(cci) * EPC);
      }
    } else {
      const int64_t cc = (c0 + scol) < dim ? (c0 + scol) : (dim - 1);
#pragma unroll
      for (int i = 0; i < NIT; ++i) {
        const int e = i * kThreads + tid;
        const int r = e / CPB;
        const int rr = r < nvalid ? r : nvalid - 1;
        const int64_t off = (b * L + t0 + rr) * dim + cc;
        xr[i] = xg[off];
        dr[i] = dg[off];
        zr[i] = zg[off];
      }
      const int nbc = nvalid * Ni;
      const int64_t base = (b * L + t0) * N;
#pragma unroll
      for (int i = 0; i < NITB; ++i) {
        const int e = i * kThreads + tid;
        const int ee = e < nbc ? e : nbc - 1;
        br[i] = Bg[base + ee];
        cr[i] = Cg[base + ee];
      }
    }
  };

  // widen one element and compute its per-(t, c) operands
  auto stage_one = [&](int idx, T xv, T dv, T zv, float Dv) {
    const float d = to_f32(dv), u = to_f32(xv);
    const float gz = has_z ? silu_gate(to_f32(zv)) : 1.f;
    Dl[idx] = d;
    Ul[idx] = d * u;
    Gl[idx] = gz;
    Yl[idx] = gz * (Dv * u);
  };

  auto stage_to_lds = [&](int64_t t0) {
    const int nvalid = static_cast<int>((t_end - t0) < TT ? (t_end - t0) : TT);
    // Register fences: the prefetched values become usable only here, so the
    // compiler cannot start consuming them (and wait for them) right after the
    // loads are issued, a tile early.
#pragma unroll
    for (int i = 0; i < NIT; ++i) asm volatile("" : "+v"(xr[i]), "+v"(dr[i]), "+v"(zr[i]));
#pragma unroll
    for (int i = 0; i < NITB; ++i) asm volatile("" : "+v"(br[i]), "+v"(cr[i]));
    if constexpr (VEC) {
#pragma unroll
      for (int i = 0; i < NIT; ++i) {
        const int idx = (i * Geo::RPI + rin) * CPB + scol;
        const T* xv = reinterpret_cast<const T*>(&xr[i]);
        const T* dv = reinterpret_cast<const T*>(&dr[i]);
        const T* zv = reinterpret_cast<const T*>(&zr[i]);
#pragma unroll
        for (int q = 0; q < EPC; ++q) stage_one(idx + q, xv[q], dv[q], has_z ? zv[q] : T(0), Dreg[q]);
      }
      const int nchunks = (nvalid * Ni) / EPC;
      const int cmask = (1 << p.bc_shift) - 1;
#pragma unroll
      for (int i = 0; i < NITB; ++i) {
        const int ci = i * kThreads + tid;
        if (ci < nchunks) {
          const int r = ci >> p.bc_shift;           // a chunk never straddles two steps
          const int n0 = (ci & cmask) * EPC;
          const T* bv = reinterpret_cast<const T*>(&br[i]);
          const T* cv = reinterpret_cast<const T*>(&cr[i]);
#pragma unroll
          for (int q = 0; q < EPC; ++q) {
            Bs[r * NP + n0 + q] = to_f32(bv[q]);
            Cs[r * NP + n0 + q] = to_f32(cv[q]);
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NIT; ++i) {
        const int e = i * kThreads + tid;
        if (e < TT * CPB) stage_one(e, xr[i], dr[i], has_z ? zr[i] : T(0), Dreg[0]);
      }
      const int nbc = nvalid * Ni;
#pragma unroll
      for (int i = 0; i < NITB; ++i) {
        const int e = i * kThreads + tid;
        if (e < nbc) {
          const int r = e / Ni, n = e - r * Ni;
          Bs[r * NP + n] = to_f32(br[i]);
          Cs[r * NP + n] = to_f32(cr[i]);
        }
      }
    }
  };

  auto store_tile = [&](int64_t t0) {
    const int nvalid = static_cast<int>((t_end - t0) < TT ? (t_end - t0) : TT);
    if constexpr (VEC) {
      const int64_t cc = c0 + scol;
#pragma unroll
      for (int i = 0; i < NIT; ++i) {
        const int r = i * Geo::RPI + rin;
        if (r < nvalid && cc < dim) {
          const uint4 v = *reinterpret_cast<const uint4*>(&ys[r * CPB + scol]);
          *reinterpret_cast<uint4*>(yg + (b * L + t0 + r) * dim + cc) = v;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NIT; ++i) {
        const int e = i * kThreads + tid;
        const int r = e / CPB;
        if (e < TT * CPB && r < nvalid && c0 + scol < dim) yg[(b * L + t0 + r) * dim + c0 + scol] = ys[e];
      }
    }
  };

  // ------------------------------------------------------------------
  // per-step work
  // ------------------------------------------------------------------
  struct Ops {
    float d, du, gz, yd;
    float b0, b1, c0, c1;           // fast path: B/C registers
    float4 bq[FAST ? 1 : NPL / 4];  // generic path: this lane's B/C values
    float4 cq[FAST ? 1 : NPL / 4];
  };
  // where this lane reads its B/C register(s) in a Bs row (fast path)
  int boff0 = 0, boff1 = 0;
  if constexpr (FAST) {
    if constexpr (G == 1) {
      boff0 = lane & 15;
    } else if constexpr (G == 2) {
      boff0 = 8 * g + (lane & 3);
      boff1 = boff0 + 4;
    } else {
      boff0 = 4 * g + (lane & 3);
    }
  }

  auto load_step = [&](int s, Ops& v) {
    v.d = Dl[s * CPB + chb];
    v.du = Ul[s * CPB + chb];
    v.gz = Gl[s * CPB + chb];
    v.yd = Yl[s * CPB + chb];
    if constexpr (FAST) {
      v.b0 = Bs[s * NP + boff0];
      v.c0 = Cs[s * NP + boff0];
      if constexpr (G == 2) {
        v.b1 = Bs[s * NP + boff1];
        v.c1 = Cs[s * NP + boff1];
      }
    } else {
      const float4* bp = reinterpret_cast<const float4*>(&Bs[s * NP + g * NPL]);
      const float4* cp = reinterpret_cast<const float4*>(&Cs[s * NP + g * NPL]);
#pragma unroll
      for (int q = 0; q < NPL / 4; ++q) {
        v.bq[q] = bp[q];
        v.cq[q] = cp[q];
      }
    }
  };

  auto do_step = [&](int s, const Ops& v) {
    float a0 = 0.f, a1 = 0.f;
    if constexpr (FAST) {
      fast_updates<G, 0, NPL>(h, A2, v.d, v.du, v.b0, G == 2 ? v.b1 : v.b0);
      if constexpr (G == 2) FastReadout<2>::run(a0, a1, v.c0, v.c1, h);
      else FastReadout<G>::run(a0, a1, v.c0, h);
    } else {
#pragma unroll
      for (int q = 0; q < NPL / 4; ++q) {
        const float bb[4] = {v.bq[q].x, v.bq[q].y, v.bq[q].z, v.bq[q].w};
        const float cc4[4] = {v.cq[q].x, v.cq[q].y, v.cq[q].z, v.cq[q].w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = q * 4 + r;
          const float dA = exp2_hw(v.d * A2[j]);
          h[j] = __builtin_fmaf(dA, h[j], v.du * bb[r]);
          if (r & 1) a1 = __builtin_fmaf(cc4[r], h[j], a1);
          else a0 = __builtin_fmaf(cc4[r], h[j], a0);
        }
      }
    }
    const float acc = reduce_groups<G, FAST>(a0 + a1);
    ys[s * CPB + chb] = from_f32<T>(__builtin_fmaf(acc, v.gz, v.yd));
    if constexpr (MODE != kSingle) {
      S += v.d;
      negseen |= (v.d < 0.f);
    }
  };

  // ------------------------------------------------------------------
  // time loop.  Per tile: stage it (waits for its loads), write the previous
  // tile's outputs from ys (other LDS arrays than the staging writes), barrier,
  // issue the next tile's loads, compute (writes ys), barrier.  Both the
  // stores and the loads thus precede the next wait by a whole tile.
  // ------------------------------------------------------------------
  if (t_begin < t_end) issue_loads(t_begin);
  int64_t prev_t0 = -1;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += TT) {
    const int ns = (t_end - t0) < TT ? static_cast<int>(t_end - t0) : TT;
    stage_to_lds(t0);
    if (prev_t0 >= 0) store_tile(prev_t0);
    __syncthreads();
    if (t0 + TT < t_end) issue_loads(t0 + TT);

    if (ns == TT) {
      // full tile: fully unrolled, operands read one step ahead (row TT is the spare zero row)
      Ops cur, nxt;
      load_step(0, cur);
#pragma unroll
      for (int s = 0; s < TT; ++s) {
        load_step(s + 1, nxt);
        do_step(s, cur);
        cur = nxt;
      }
    } else {
      Ops va, vb;
      load_step(0, va);
      int s = 0;
      for (; s + 1 < ns; s += 2) {
        load_step(s + 1, vb);
        do_step(s, va);
        load_step(s + 2, va);     // row s + 2 <= ns < TT: loaded, never used
        do_step(s + 1, vb);
      }
      if (s < ns) do_step(s, va);
    }
    __syncthreads();
    prev_t0 = t0;

    if constexpr (MODE == kFixup) {
      // carried-in part bounded by exp2(amax * S) * hmax; done once it would be 0 in fp32
      const bool lane_done = !cvalid || hmax == 0.f ||
                             (!never_exit && amax < 0.f && amax * S + __log2f(hmax) < -150.f);
      if (__syncthreads_and(lane_done)) break;
    }
  }
  if (prev_t0 >= 0) store_tile(prev_t0);

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

// ---------------------------------------------------------------------------
// One state per lane ("wide" layout), dstate == 16.
//
// A 16-lane row of a wave is one channel and lane n of the row holds its state
// n, so a problem has 16 lanes per channel and fills the chip with several
// waves per SIMD even where batch * dim is small.  Per step a lane issues five
// VALU operations and nothing else: delta and delta*x of step s come from lane
// s of its row (row_newbcast:s, folded by the compiler into v_mul_f32_dpp),
// B_n and C_n are the lane's own registers (read from transposed LDS copies,
// 16-byte reads covering 4 steps).  The readout's sum over the 16 states runs
// once per 16 steps: lanes n and n+8 add their 16 products C_n h_n with a DPP
// row rotation, lanes 0-7 park those pair sums in LDS, and each lane reads
// back the 8 pair sums of one step (a transpose), so lane j of a row finishes
// step j, applies the gate and writes the output.  Steps past the end of the
// sequence are staged with delta = 0, which leaves the state unchanged exactly
// (exp2(0) = 1, delta*x = 0).
// ---------------------------------------------------------------------------
namespace wide {
constexpr int CPB = 16;            // channels per block (one per 16-lane row)
constexpr int TT = 64;             // steps per tile (4 groups of 16)
constexpr int QS = TT + 1;         // float4 row stride of the per-(c, t) operands (spreads banks)
constexpr int BS = TT + 4;         // float row stride of the transposed B/C tiles
constexpr int PS = 20;             // float stride between one lane's 16 pair sums
constexpr int PR = 8 * PS + 16;    // float stride between rows of the pair-sum buffer (16 mod 32: rows on other banks)
}  // namespace wide

using u32x2 = unsigned int __attribute__((ext_vector_type(2)));

template <int S> __device__ __forceinline__ float row_bcast(float v) { return dpp<row_newbcast(S)>(v); }

// 16 recurrence steps of one lane: its state h, exponent slope a2, the step
// operands q (delta, delta*x held by lane s of the row for step s), B_n and
// C_n per step; products C_n h_n land in pr.
template <int S>
__device__ __forceinline__ void wide_steps(float& h, float a2, float qd, float qu, const float (&Bv)[16],
                                           const float (&Cv)[16], float (&pr)[16]) {
  const float dA = exp2_hw(row_bcast<S>(qd) * a2);
  h = __builtin_fmaf(dA, h, row_bcast<S>(qu) * Bv[S]);
  pr[S] = Cv[S] * h;
  if constexpr (S + 1 < 16) wide_steps<S + 1>(h, a2, qd, qu, Bv, Cv, pr);
}

__device__ __forceinline__ float row_sum(float v) {
  v += dpp<0x128>(v);   // row_ror:8
  v += dpp<0x124>(v);   // row_ror:4
  v += dpp<0x122>(v);   // row_ror:2
  v += dpp<0x121>(v);   // row_ror:1
  return v;
}

// variants of the one-state-per-lane kernel
constexpr int kPlain = 0;   // the scan
constexpr int kConv = 1;    // short causal convolution + SiLU in front (x from its input)
constexpr int kCkpt = 2;    // training mode: also store the state entering every 16-step tile

template <int IO, int MODE, int VAR>
__global__ __launch_bounds__(kThreads) void wide_kernel(KernelParams p) {
  constexpr bool CONV = VAR == kConv;
  using namespace wide;
  using T = typename IoType<IO>::T;
  // a staging thread moves 4 channels (or 4 states of B/C) of one step
  using Chunk = typename std::conditional<IO == 1, u32x2, u32x4>::type;

  __shared__ __attribute__((aligned(16))) float4 Qs[CPB * QS];      // {delta, delta*x, silu(z), silu(z)*D*x} [c][t]
  __shared__ __attribute__((aligned(16))) float Bt[16 * BS];        // B [n][t]
  __shared__ __attribute__((aligned(16))) float Ct[16 * BS];        // C [n][t]
  __shared__ __attribute__((aligned(16))) float Pb[kThreads / 16 * PR];   // per-row products [row][n][s]
  __shared__ __attribute__((aligned(16))) T ys[TT * CPB];           // outputs of the previous tile [t][c]

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int row = tid / 16;            // channel within the block (4 rows per wave)
  const int n = lane % 16;             // state of this lane; also the step it finishes in a group

  // block -> (batch, chunk, channel group); 4 consecutive channel groups (one
  // 128-byte line of a bf16 row) run on one XCD, whose L2 then serves them all
  const int64_t nb = gridDim.x;
  const int64_t bid = blockIdx.x;
  int64_t lin = bid;
  if (bid < (nb / 32) * 32) {
    const int64_t xcd = bid % 8, rr = bid / 8;
    lin = ((rr / 4) * 8 + xcd) * 4 + rr % 4;
  }
  const int cg = static_cast<int>(lin % p.ngroups);
  const int64_t rest = lin / p.ngroups;
  const int nchunks_here = (MODE == kFixup) ? p.K - 1 : p.K;
  const int k = static_cast<int>(rest % nchunks_here) + p.chunk_offset;
  const int64_t b = rest / nchunks_here;

  const int64_t dim = p.dim, L = p.L;
  const int64_t c0 = static_cast<int64_t>(cg) * CPB;
  const int64_t c = c0 + row;
  const bool cvalid = c < dim;
  const int64_t cl = cvalid ? c : dim - 1;
  const int64_t t_begin = static_cast<int64_t>(k) * p.chunk_len;
  const int64_t t_end = t_begin + p.chunk_len < L ? t_begin + p.chunk_len : L;

  const T* __restrict__ xg = static_cast<const T*>(p.x);
  const T* __restrict__ dg = static_cast<const T*>(p.delta);
  const T* __restrict__ zg = static_cast<const T*>(p.z != nullptr ? p.z : p.x);
  const T* __restrict__ Bg = static_cast<const T*>(p.B);
  const T* __restrict__ Cg = static_cast<const T*>(p.C);
  T* __restrict__ yg = static_cast<T*>(p.out);
  const bool has_z = p.z != nullptr;

  const float a2 = p.A[cl * 16 + n] * kLog2e;
  float h = 0.f;
  if constexpr (MODE == kFixup) {
    h = p.hin[((b * p.K + k) * dim + cl) * 16 + n];
  } else {
    if (p.h0 != nullptr && (MODE == kSingle || k == 0)) h = p.h0[(b * dim + cl) * 16 + n];
  }
  const float h_in = h;
  bool never_exit = false;
  if constexpr (MODE == kFixup) never_exit = p.neg[(b * p.K + k) * dim + cl] != 0;
  float S = 0.f;         // this lane's share of the chunk's delta sum (the steps it stages)
  float negseen = 0.f;   // 1 once a negative delta was seen among those steps

  // staging: thread -> (step ts, 4 channels / states from 4*q4)
  const int ts = tid / 4, q4 = tid % 4;
  const int64_t sc = (c0 + 4 * q4) < dim ? (c0 + 4 * q4) : (dim - 4);   // dim % 4 == 0
  float Dreg[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) Dreg[q] = p.D != nullptr ? p.D[sc + q] : 0.f;

  // Short causal convolution (CONV): the staging thread's 4 channels need the
  // input at steps t-3 .. t.  Taps are right-aligned into 4 slots (slot 3 =
  // step t), so a narrower kernel has leading zero taps; the block's taps and
  // biases sit in LDS.  Steps before 0 come from conv_init (or are 0).
  __shared__ float4 Wl[CONV ? CPB : 1];   // taps of the block's channels
  __shared__ float Bl[CONV ? CPB : 1];    // biases
  Chunk xh[3];            // input at t-1, t-2, t-3
  bool hvalid[3];
  if constexpr (CONV) {
    if (tid < CPB) {
      const int W = p.conv_width;
      const int64_t cc = c0 + tid;
      float tap[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) tap[k] = (cc < dim && k >= 4 - W) ? p.conv_w[cc * W + (k - (4 - W))] : 0.f;
      Wl[tid] = float4{tap[0], tap[1], tap[2], tap[3]};
      Bl[tid] = (cc < dim && p.conv_b != nullptr) ? p.conv_b[cc] : 0.f;
    }
    __syncthreads();
  }

  Chunk xr, dr, zr, br, cr;
  auto issue_loads = [&](int64_t t0) {
    const int nvalid = static_cast<int>((t_end - t0) < TT ? (t_end - t0) : TT);
    const int rr = ts < nvalid ? ts : nvalid - 1;
    const int64_t row_t = b * L + t0 + rr;
    if constexpr (CONV) {
      const T* ig = static_cast<const T*>(p.conv_init);
      const int W = p.conv_width;
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int64_t tt = t0 + rr - (j + 1);
        const bool from_init = tt < 0 && ig != nullptr && (W - 1) + tt >= 0;
        hvalid[j] = tt >= 0 || from_init;
        // always an in-range address; the value is masked at staging when not valid
        const T* src = tt >= 0 ? xg + (row_t - (j + 1)) * dim + sc
                               : (from_init ? ig + (b * (W - 1) + (W - 1) + tt) * dim + sc : xg + b * L * dim + sc);
        xh[j] = *reinterpret_cast<const Chunk*>(src);
      }
    }
    xr = *reinterpret_cast<const Chunk*>(xg + row_t * dim + sc);
    dr = *reinterpret_cast<const Chunk*>(dg + row_t * dim + sc);
    zr = *reinterpret_cast<const Chunk*>(zg + row_t * dim + sc);
    br = *reinterpret_cast<const Chunk*>(Bg + row_t * 16 + 4 * q4);
    cr = *reinterpret_cast<const Chunk*>(Cg + row_t * 16 + 4 * q4);
  };

  auto stage = [&](int64_t t0) {
    const int nvalid = static_cast<int>((t_end - t0) < TT ? (t_end - t0) : TT);
    asm volatile("" : "+v"(xr), "+v"(dr), "+v"(zr), "+v"(br), "+v"(cr));
    float ux[4];   // the scan's x of the 4 channels at this step
    if constexpr (CONV) {
      asm volatile("" : "+v"(xh[0]), "+v"(xh[1]), "+v"(xh[2]));
      const T* x0 = reinterpret_cast<const T*>(&xr);
      const T* x1 = reinterpret_cast<const T*>(&xh[0]);
      const T* x2 = reinterpret_cast<const T*>(&xh[1]);
      const T* x3 = reinterpret_cast<const T*>(&xh[2]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 w = Wl[4 * q4 + q];
        float a = __builtin_fmaf(w.w, to_f32(x0[q]), Bl[4 * q4 + q]);
        a = __builtin_fmaf(w.z, hvalid[0] ? to_f32(x1[q]) : 0.f, a);
        a = __builtin_fmaf(w.y, hvalid[1] ? to_f32(x2[q]) : 0.f, a);
        a = __builtin_fmaf(w.x, hvalid[2] ? to_f32(x3[q]) : 0.f, a);
        ux[q] = silu_gate(a);
      }
    } else {
      const T* xv0 = reinterpret_cast<const T*>(&xr);
#pragma unroll
      for (int q = 0; q < 4; ++q) ux[q] = to_f32(xv0[q]);
    }
    const T* dv = reinterpret_cast<const T*>(&dr);
    const T* zv = reinterpret_cast<const T*>(&zr);
    const T* bv = reinterpret_cast<const T*>(&br);
    const T* cv = reinterpret_cast<const T*>(&cr);
    // steps past the end (last tile only) get delta = 0: an exact no-op step
    const float keep = ts < nvalid ? 1.f : 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float d = to_f32(dv[q]), u = ux[q];
      const float gz = has_z ? silu_gate(to_f32(zv[q])) : 1.f;
      float4 v = float4{d, d * u, gz, gz * (Dreg[q] * u)};
      if (nvalid < TT) v = float4{v.x * keep, v.y * keep, v.z * keep, v.w * keep};
      Qs[(4 * q4 + q) * QS + ts] = v;
      Bt[(4 * q4 + q) * BS + ts] = to_f32(bv[q]);
      Ct[(4 * q4 + q) * BS + ts] = to_f32(cv[q]);
    }
  };

  auto store_tile = [&](int64_t t0) {
    const int nvalid = static_cast<int>((t_end - t0) < TT ? (t_end - t0) : TT);
    // TT rows of 16 channels: 16 / (16 / sizeof(T)) 16-byte pieces per row
    constexpr int PPR = CPB * static_cast<int>(sizeof(T)) / 16;
    for (int e = tid; e < TT * PPR; e += kThreads) {
      const int rrow = e / PPR, piece = e % PPR;
      const int64_t cc = c0 + piece * (16 / static_cast<int>(sizeof(T)));
      if (rrow < nvalid && cc < dim)
        *reinterpret_cast<u32x4*>(yg + (b * L + t0 + rrow) * dim + cc) =
            *reinterpret_cast<const u32x4*>(&ys[rrow * CPB + piece * (16 / static_cast<int>(sizeof(T)))]);
    }
  };

  float* const Prow = &Pb[row * PR];

  // operands of one 16-step group: q = {delta, delta*x, silu(z), silu(z)*D*x}
  // of step t16 + n, and B_n, C_n of the 16 steps
  struct GroupOps {
    float4 q;
    float Bv[16], Cv[16];
  };
  auto load_ops = [&](int t16, GroupOps& o) {
    o.q = Qs[row * QS + t16 + n];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 bb = *reinterpret_cast<const float4*>(&Bt[n * BS + t16 + 4 * i]);
      const float4 cc = *reinterpret_cast<const float4*>(&Ct[n * BS + t16 + 4 * i]);
      o.Bv[4 * i] = bb.x; o.Bv[4 * i + 1] = bb.y; o.Bv[4 * i + 2] = bb.z; o.Bv[4 * i + 3] = bb.w;
      o.Cv[4 * i] = cc.x; o.Cv[4 * i + 1] = cc.y; o.Cv[4 * i + 2] = cc.z; o.Cv[4 * i + 3] = cc.w;
    }
  };
  // transpose through LDS (issued here, summed later so the LDS latency
  // overlaps the next group's arithmetic).  First lanes n and n+8 of a row add
  // their 16 products (row_ror:8), which halves the bytes moved through LDS:
  // both lanes then hold the same sums, lanes 0-7 park them, and each lane
  // reads the 8 pair sums of its step.
  auto park_and_fetch = [&](const float (&pr)[16], float (&rd)[8]) {
    float ps[16];
    {
      // one v_add_f32_dpp per product with every lane active: the add must not be contracted into
      // an FMA with the product (that leaves the DPP move unfolded), and the sums are pinned before
      // the branch below (inside it the DPP could not be folded either)
#pragma clang fp contract(off)
#pragma unroll
      for (int i = 0; i < 16; ++i) ps[i] = pr[i] + dpp_bc<kRowRor8>(pr[i]);
    }
    asm volatile("" : "+v"(ps[0]), "+v"(ps[1]), "+v"(ps[2]), "+v"(ps[3]), "+v"(ps[4]), "+v"(ps[5]), "+v"(ps[6]),
                 "+v"(ps[7]));
    asm volatile("" : "+v"(ps[8]), "+v"(ps[9]), "+v"(ps[10]), "+v"(ps[11]), "+v"(ps[12]), "+v"(ps[13]),
                 "+v"(ps[14]), "+v"(ps[15]));
    if (n < 8) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<float4*>(&Prow[n * PS + 4 * i]) = float4{ps[4 * i], ps[4 * i + 1], ps[4 * i + 2], ps[4 * i + 3]};
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int m = 0; m < 8; ++m) rd[m] = Prow[m * PS + n];
    __builtin_amdgcn_wave_barrier();
  };
  auto finish = [&](int t16, const float4& q, const float (&rd)[8]) {
    const float y = ((rd[0] + rd[1]) + (rd[2] + rd[3])) + ((rd[4] + rd[5]) + (rd[6] + rd[7]));
    ys[(t16 + n) * CPB + row] = from_f32<T>(__builtin_fmaf(y, q.z, q.w));
    if constexpr (MODE != kSingle) {
      S += q.x;
      negseen = q.x < 0.f ? 1.f : negseen;
    }
  };
  // one group start to finish (tail tiles)
  // training mode: store the state entering the 16-step group at tile step t16
  // (chunks start on 16-step boundaries, so it is a whole checkpoint tile)
  int64_t cur_t0 = t_begin;
  auto checkpoint = [&](int t16) {
    if constexpr (VAR == kCkpt) {
      if (cvalid) {
        const int64_t kt = (cur_t0 + t16) / 16;
        p.ckpt[((b * p.ckpt_tiles + kt) * (16 * static_cast<int64_t>(p.ngroups)) + c) * 16 + n] = h;
      }
    }
  };
  auto group = [&](int t16) {
    GroupOps o;
    float pr[16], rd[8];
    load_ops(t16, o);
    checkpoint(t16);
    wide_steps<0>(h, a2, o.q.x, o.q.y, o.Bv, o.Cv, pr);
    park_and_fetch(pr, rd);
    finish(t16, o.q, rd);
  };
  // a full tile, software-pipelined: group g+1's operands are read before
  // group g's steps, group g-1's sum after them
  auto full_tile = [&]() {
    GroupOps o[2];
    float pr[16], rd[8];
    float4 qprev;
    load_ops(0, o[0]);
#pragma unroll
    for (int g = 0; g < TT / 16; ++g) {
      if (g + 1 < TT / 16) load_ops(16 * (g + 1), o[(g + 1) & 1]);
      checkpoint(16 * g);
      wide_steps<0>(h, a2, o[g & 1].q.x, o[g & 1].q.y, o[g & 1].Bv, o[g & 1].Cv, pr);
      if (g > 0) finish(16 * (g - 1), qprev, rd);
      park_and_fetch(pr, rd);
      qprev = o[g & 1].q;
    }
    finish(TT - 16, qprev, rd);
  };

  if (t_begin < t_end) issue_loads(t_begin);
  int64_t prev_t0 = -1;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += TT) {
    const int ns = (t_end - t0) < TT ? static_cast<int>(t_end - t0) : TT;
    cur_t0 = t0;
    stage(t0);
    if (prev_t0 >= 0) store_tile(prev_t0);
    __syncthreads();
    if (t0 + TT < t_end) issue_loads(t0 + TT);
    if (ns == TT) {
      full_tile();
    } else {
      for (int t16 = 0; t16 < ns; t16 += 16) group(t16);
    }
    __syncthreads();
    prev_t0 = t0;
    if constexpr (MODE == kFixup) {
      // state n's carried-in part is exp2(a2 * sum(delta)) * h_in; done once it is 0 in fp32
      const float Srow = row_sum(S);
      const bool lane_done = !cvalid || h_in == 0.f ||
                             (!never_exit && a2 < 0.f && a2 * Srow + __log2f(fabsf(h_in)) < -150.f);
      if (__syncthreads_and(lane_done)) break;
    }
  }
  if (prev_t0 >= 0) store_tile(prev_t0);

  if constexpr (MODE == kSingle) {
    if (p.final_state != nullptr && cvalid) p.final_state[(b * dim + c) * 16 + n] = h;
  } else if constexpr (MODE == kChunk) {
    const float Srow = row_sum(S);
    float ng = negseen;
    ng = fmaxf(ng, dpp<0x128>(ng));
    ng = fmaxf(ng, dpp<0x124>(ng));
    ng = fmaxf(ng, dpp<0x122>(ng));
    ng = fmaxf(ng, dpp<0x121>(ng));
    if (cvalid) {
      p.hend[((b * p.K + k) * dim + c) * 16 + n] = h;
      if (n == 0) {
        p.S[(b * p.K + k) * dim + c] = Srow;
        p.neg[(b * p.K + k) * dim + c] = ng > 0.f ? 1 : 0;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// One channel per lane, every wave on its own ("lane" layout), dstate == 16.
//
// A wave owns 64 consecutive channels of one batch row and one sequence chunk,
// and lane c holds the 16 states of channel c in VGPRs; with bf16 I/O a
// workgroup is eight such waves (two on every SIMD), with fp32 one.  Waves
// share no data, so there is no barrier: each wave copies its own
// time tiles of x, delta, z and of B, C from HBM into its LDS with direct
// global->LDS loads (one tile ahead, double-buffered) and lane c reads the
// values of its channel at step s from there.  B_n and C_n reach the lanes as
// in the one-lane-per-channel fast path above: lane n of each 16-lane row
// reads state n's value and the update and readout take it through a DPP
// row_newbcast operand.  Per step a lane does the 16 updates, the readout and
// the per-(t, c) work of its own channel (widening, delta*x, the SiLU gate,
// D*x); outputs collect in an LDS tile that is written back with 16-byte
// stores at the start of the next tile.
//
// Ordering of the direct loads: a tile's loads are issued before the previous
// tile is computed, and the wait before a tile is computed lets only the loads
// issued after them (the next tile's) stay in flight.  Every vector-memory
// operation issued earlier (the output stores of two tiles back) has then
// completed as well, since the counter retires in issue order.
// ---------------------------------------------------------------------------
namespace lanek {
constexpr int TT = 16;   // steps per tile
// waves per workgroup: with bf16 eight (16 KB of LDS each, 128 KB, two waves on every SIMD of the CU);
// fp32 tiles take 32 KB a wave, so one wave per workgroup
constexpr int wpb(int io) { return io == 1 ? 8 : 1; }
}

__device__ __forceinline__ uint32_t lds_off(const void* p) {
  // the low half of a flat address into LDS is the LDS offset
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}
// global -> LDS: lane l's 16 bytes land at LDS offset lds + 16 l (lds is wave-uniform and goes to M0).
// Written as asm with no outputs, so the compiler neither tracks nor waits for these loads and no
// register can be overwritten while one is in flight; completion is waited for with wait_vmcnt.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
// wait until at most n (0..15, wave-uniform) of this wave's vector-memory operations are outstanding
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case 15: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
    case 14: asm volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
    case 13: asm volatile("s_waitcnt vmcnt(13)" ::: "memory"); break;
    case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 11: asm volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
    case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

// 8 bytes of a transposing LDS read (ds_read_b64_tr_b16); the element layout is at its use
__device__ __forceinline__ u32x2 tr_read(const unsigned char* p) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const_cast<unsigned char*>(p)));
  return __builtin_bit_cast(u32x2, v);
}

template <int IO, int MODE>
__global__ __launch_bounds__(kWave * lanek::wpb(IO)) void lane_kernel(KernelParams p) {
  using namespace lanek;
  using T = typename IoType<IO>::T;
  constexpr int ES = sizeof(T);
  constexpr int EPC = 16 / ES;                    // elements per 16-byte piece
  constexpr int RBY = kWave * ES;                 // bytes of one step of the wave's 64 channels
  constexpr int TB = TT * RBY;                    // bytes of one tensor's tile
  constexpr int NX = TB / 1024;                   // 16-byte loads per lane for one tensor's tile
  constexpr int PPR = RBY / 16;                   // 16-byte pieces per step row
  constexpr int RPI = kWave / PPR;                // step rows per load instruction
  constexpr int BCB = TT * 16 * ES;               // bytes of B (or of C) per tile
  constexpr int BCW = BCB / 16;                   // 16-byte pieces of B (or C) per tile
  constexpr int NBC = (2 * BCB + 1023) / 1024;    // 16-byte loads per lane for B and C together
  static_assert(TB % 1024 == 0 && BCB % 16 == 0, "tile geometry");

  constexpr int WPB = wpb(IO);
  __shared__ __attribute__((aligned(16))) unsigned char xs_[WPB][2][TB];
  __shared__ __attribute__((aligned(16))) unsigned char dls_[WPB][2][TB];
  __shared__ __attribute__((aligned(16))) unsigned char zs_[WPB][2][TB];
  __shared__ __attribute__((aligned(16))) unsigned char bcs_[WPB][2][NBC * 1024];   // B [t][n], then C [t][n]
  __shared__ __attribute__((aligned(16))) T ys_[WPB][TT * kWave];                   // outputs [t][c]
  __shared__ int prog[WPB];   // tiles each wave has finished (INT_MAX: no more work)

  const int lane = threadIdx.x % kWave;
  const int w = WPB > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x / kWave) : 0;
  auto& xs = xs_[w];
  auto& dls = dls_[w];
  auto& zs = zs_[w];
  auto& bcs = bcs_[w];
  T* const ys = &ys_[w][0];
  const int64_t bid = static_cast<int64_t>(blockIdx.x) * WPB + w;   // this wave's unit
  const int nunits_k = (MODE == kFixup) ? p.K - 1 : p.K;
  const bool idle = bid >= p.batch * nunits_k * p.ngroups;   // a wave past the last unit of the grid
  if constexpr (WPB > 1) {
    if (lane == 0) prog[w] = idle ? INT_MAX : 0;
    __syncthreads();
  }
  if (idle) return;
  const int cg = static_cast<int>(bid % p.ngroups);
  const int64_t rest = bid / p.ngroups;
  const int nchunks_here = (MODE == kFixup) ? p.K - 1 : p.K;
  const int k = static_cast<int>(rest % nchunks_here) + p.chunk_offset;
  const int64_t b = rest / nchunks_here;

  const int64_t dim = p.dim, L = p.L;
  const int64_t c0 = static_cast<int64_t>(cg) * kWave;
  const int64_t c = c0 + lane;
  const bool cvalid = c < dim;
  const int64_t cl = cvalid ? c : dim - 1;
  const int64_t t_begin = static_cast<int64_t>(k) * p.chunk_len;
  const int64_t t_end = t_begin + p.chunk_len < L ? t_begin + p.chunk_len : L;

  const T* __restrict__ xg = static_cast<const T*>(p.x);
  const T* __restrict__ dg = static_cast<const T*>(p.delta);
  const T* __restrict__ zg = static_cast<const T*>(p.z);
  const T* __restrict__ Bg = static_cast<const T*>(p.B);
  const T* __restrict__ Cg = static_cast<const T*>(p.C);
  T* __restrict__ yg = static_cast<T*>(p.out);
  const bool has_z = p.z != nullptr;

  float A2[16], h[16];
  float amax = -INFINITY;   // largest (least negative) exponent slope of the channel
  float hmax = 0.f;         // largest |h_in| (fix-up)
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    A2[j] = cvalid ? p.A[c * 16 + j] * kLog2e : 0.f;
    float h_init = 0.f;
    if constexpr (MODE == kFixup) {
      h_init = cvalid ? p.hin[((b * p.K + k) * dim + c) * 16 + j] : 0.f;
    } else {
      if (p.h0 != nullptr && cvalid && (MODE == kSingle || k == 0)) h_init = p.h0[(b * dim + c) * 16 + j];
    }
    h[j] = h_init;
    if (cvalid) {
      amax = fmaxf(amax, A2[j]);
      hmax = fmaxf(hmax, fabsf(h_init));
    }
  }
  bool never_exit = false;
  if constexpr (MODE == kFixup) never_exit = cvalid && p.neg[(b * p.K + k) * dim + c] != 0;
  const float Dv = p.D != nullptr ? p.D[cl] : 0.f;
  float S = 0.f;
  int negseen = 0;

  // this lane's 16-byte piece of a step row: row lane / PPR of each load, channels from pc
  const int lrow = lane / PPR;
  int64_t pc = c0 + (lane % PPR) * EPC;
  if (pc > dim - EPC) pc = dim - EPC;   // dim is a multiple of EPC; pieces past the end repeat the last one
  const int nload = NX * (has_z ? 3 : 2) + NBC;

  // all of a tile's loads, unconditionally (rows past the chunk end repeat its last step)
  auto issue = [&](int64_t t0, int buf) {
    const int64_t nv = (t_end - t0) < TT ? (t_end - t0) : TT;
#pragma unroll
    for (int j = 0; j < NX; ++j) {
      const int64_t r = j * RPI + lrow;
      const int64_t off = (b * L + t0 + (r < nv ? r : nv - 1)) * dim + pc;
      lds_dma16(xg + off, lds_off(&xs[buf][0]) + j * 1024);
      lds_dma16(dg + off, lds_off(&dls[buf][0]) + j * 1024);
      if (has_z) lds_dma16(zg + off, lds_off(&zs[buf][0]) + j * 1024);
    }
#pragma unroll
    for (int j = 0; j < NBC; ++j) {
      int g = j * kWave + lane, tsr = g / BCW, w = g % BCW;
      if (tsr > 1) {   // spare lanes of the last load: repeat C's last piece into the spare LDS space
        tsr = 1;
        w = BCW - 1;
      }
      const int64_t r = w / ES;   // ES pieces per step row of 16 states
      const int64_t off = (b * L + t0 + (r < nv ? r : nv - 1)) * 16 + (w % ES) * EPC;
      lds_dma16((tsr ? Cg : Bg) + off, lds_off(&bcs[buf][0]) + j * 1024);
    }
  };

  // one step from its widened values (zv: z, read only when HZ)
  auto step_v = [&](auto hz, int s, float d, float u, float zv, float bv, float cv) {
    constexpr bool HZ = decltype(hz)::value;
    fast_updates<1, 0, 16>(h, A2, d, d * u, bv, bv);
    float a0, a1;
    FastReadout<1>::run(a0, a1, cv, h);
    float y = a0 + a1;
    if constexpr (HZ) {
      y = __builtin_fmaf(Dv, u, y) * silu_gate(zv);
    } else {
      y = __builtin_fmaf(Dv, u, y);
    }
    ys[s * kWave + lane] = from_f32<T>(y);
    if constexpr (MODE != kSingle) {
      S += d;
      negseen |= (d < 0.f);
    }
  };
  // HZ: z is given (a compile-time copy of has_z, so that a tile is one straight block of code)
  auto step = [&](auto hz, int buf, int s) {
    constexpr bool HZ = decltype(hz)::value;
    const float d = to_f32(*reinterpret_cast<const T*>(&dls[buf][s * RBY + lane * ES]));
    const float u = to_f32(*reinterpret_cast<const T*>(&xs[buf][s * RBY + lane * ES]));
    const float bv = to_f32(*reinterpret_cast<const T*>(&bcs[buf][(s * 16 + (lane & 15)) * ES]));
    const float cv = to_f32(*reinterpret_cast<const T*>(&bcs[buf][BCB + (s * 16 + (lane & 15)) * ES]));
    const float zv = HZ ? to_f32(*reinterpret_cast<const T*>(&zs[buf][s * RBY + lane * ES])) : 0.f;
    step_v(hz, s, d, u, zv, bv, cv);
  };
  // Four steps from five transposing LDS reads (bf16 only).  In each 16-lane group, lanes 4k..4k+3
  // point at four consecutive 2-byte elements of row s0 + k and lane j receives element j of each
  // row k = 0..3.  For x, delta and z the group's 16 elements are its 16 channels, so lane c gets its
  // channel's values of steps s0..s0+3; for B and C they are the 16 states, so lane n of every row gets
  // B_n and C_n of those steps, where the DPP operands of the updates and the readout take them from.
  const int tr_k = (lane & 15) >> 2, tr_i = lane & 3;
  const int tr_x = tr_k * RBY + 32 * (lane >> 4) + 8 * tr_i;   // + s0 * RBY
  const int tr_b = tr_k * 32 + 8 * tr_i;                        // + s0 * 32 (B), + BCB (C)
  auto quad = [&](auto hz, int buf, int s0) {
    constexpr bool HZ = decltype(hz)::value;
    const u32x2 dq = tr_read(&dls[buf][s0 * RBY + tr_x]);
    const u32x2 xq = tr_read(&xs[buf][s0 * RBY + tr_x]);
    const u32x2 bq = tr_read(&bcs[buf][s0 * 32 + tr_b]);
    const u32x2 cq = tr_read(&bcs[buf][BCB + s0 * 32 + tr_b]);
    u32x2 zq = u32x2{0u, 0u};
    if constexpr (HZ) zq = tr_read(&zs[buf][s0 * RBY + tr_x]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t sh = (k & 1) ? 0u : 16u;
      const uint32_t mk = (k & 1) ? 0xffff0000u : 0xffffffffu;
      auto wid = [&](const u32x2& q) { return __uint_as_float((q[k >> 1] << sh) & mk); };
      step_v(hz, s0 + k, wid(dq), wid(xq), HZ ? wid(zq) : 0.f, wid(bq), wid(cq));
    }
  };

  // the outputs of the tile at t0 from ys: 16-byte pieces, rows past the chunk end skipped
  auto store_tile = [&](int64_t t0) {
    const int64_t nv = (t_end - t0) < TT ? (t_end - t0) : TT;
#pragma unroll
    for (int j = 0; j < NX; ++j) {
      const int r = j * RPI + lrow;
      const int64_t cc = c0 + (lane % PPR) * EPC;
      const u32x4 v = *reinterpret_cast<const u32x4*>(&ys[r * kWave + (lane % PPR) * EPC]);
      if (r < nv && cc < dim) *reinterpret_cast<u32x4*>(yg + (b * L + t0 + r) * dim + cc) = v;
    }
  };

  // The waves of a workgroup with the same w % 4 share a SIMD.  The SIMD issues from the older of two ready
  // waves, so left alone one wave of a pair runs ahead and the other finishes its chunk alone, at the
  // lower issue rate of a single wave.  At each tile a wave takes priority 0 when it has finished more
  // tiles than its partner, 2 when fewer and 1 when as many, which keeps the pair within about a tile.
  auto pace = [&](int i) {
    int other = INT_MAX;
#pragma unroll
    for (int m = 1; m < WPB / 4; ++m)
      other = min(other, __hip_atomic_load(&prog[(w + 4 * m) % WPB], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
    __hip_atomic_store(&prog[w], i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (i > other) __builtin_amdgcn_s_setprio(0);
    else if (i == other) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(2);
  };
  auto run = [&](auto hz) {
    int64_t prev_t0 = -1;
    int i = 0;
    if (t_begin < t_end) issue(t_begin, 0);
    for (int64_t t0 = t_begin; t0 < t_end; t0 += TT, ++i) {
      const int buf = i & 1;
      int inflight = 0;
      if (t0 + TT < t_end) {
        issue(t0 + TT, buf ^ 1);
        inflight = nload;
      }
      wait_vmcnt(inflight);
      if constexpr (WPB > 1) pace(i);
      if (prev_t0 >= 0) store_tile(prev_t0);
      const int64_t ns = (t_end - t0) < TT ? (t_end - t0) : TT;
      if (ns == TT) {
        if constexpr (ES == 2) {
#pragma unroll
          for (int s0 = 0; s0 < TT; s0 += 4) quad(hz, buf, s0);
        } else {
#pragma unroll
          for (int s = 0; s < TT; ++s) step(hz, buf, s);
        }
      } else {
        for (int s = 0; s < static_cast<int>(ns); ++s) step(hz, buf, s);
      }
      prev_t0 = t0;
      if constexpr (MODE == kFixup) {
        // The carried-in part of state j is bounded by exp2(A2[j] S) hmax.  Done once it would be 0 in
        // fp32, or once it is below 2^-26 of every state it is part of: from there on the zero-start
        // values the chunk pass stored differ from the rescanned ones only by fp32 rounding of the states.
        bool below = true;
#pragma unroll
        for (int j = 0; j < 16; ++j) below = below && exp2_hw(A2[j] * S) * hmax < 0x1p-26f * fabsf(h[j]);
        const bool lane_done = !cvalid || hmax == 0.f ||
                               (!never_exit && amax < 0.f && (amax * S + __log2f(hmax) < -150.f || below));
        if (__builtin_amdgcn_ballot_w64(!lane_done) == 0) break;
      }
    }
    if (prev_t0 >= 0) store_tile(prev_t0);
    wait_vmcnt(0);   // a fix-up wave can leave with the next tile's loads in flight
    if constexpr (WPB > 1) {
      __hip_atomic_store(&prog[w], INT_MAX, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);   // never hold the partner back
      __builtin_amdgcn_s_setprio(0);
    }
  };
  if (has_z) run(std::true_type{});
  else run(std::false_type{});

  if constexpr (MODE == kSingle) {
    if (p.final_state != nullptr && cvalid) {
#pragma unroll
      for (int j = 0; j < 16; ++j) p.final_state[(b * dim + c) * 16 + j] = h[j];
    }
  } else if constexpr (MODE == kChunk) {
    if (cvalid) {
#pragma unroll
      for (int j = 0; j < 16; ++j) p.hend[((b * p.K + k) * dim + c) * 16 + j] = h[j];
      p.S[(b * p.K + k) * dim + c] = S;
      p.neg[(b * p.K + k) * dim + c] = negseen;
    }
  }
}

// Carry across chunks, as a wave-level parallel scan over the chunks' affine maps.
// Chunk k >= 1 takes the state entering it to the state leaving it by
//   h -> a_k h + hend_k,   a_k = exp2(A' S_k)   (hend_k: its end state from a zero start),
// and two consecutive maps compose as (a1, b1) then (a2, b2) = (a1 a2, a2 b1 + b2), which is
// associative ("03 - Modelos de espacio de estados", "Parallel scan").  One wave per (b, c, n):
// lane j holds the m = ceil((K-1)/64) consecutive chunks from 1 + j m and composes them in order,
// the wave scans the 64 lane maps in log2(64) = 6 shuffle steps, and each lane applies its
// exclusive prefix to the true end state of chunk 0, then walks its chunks again writing h_in.
__global__ __launch_bounds__(256) void carry_kernel(KernelParams p) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t col = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / kWave;
  if (col >= p.batch * p.dim * p.N) return;   // col is uniform within a wave: whole waves leave
  const int64_t n = col % p.N;
  const int64_t c = (col / p.N) % p.dim;
  const int64_t b = col / (p.N * p.dim);
  const float a2 = p.A[c * p.N + n] * kLog2e;
  const int K = p.K;
  const int m = (K - 1 + kWave - 1) / kWave;
  const int k_lo = 1 + lane * m;
  const int k_hi = k_lo + m < K ? k_lo + m : K;
  const float* __restrict__ S = p.S + b * K * p.dim + c;                // S[k * dim]
  const float* __restrict__ he = p.hend + (b * K * p.dim + c) * p.N + n;   // hend[k * dim * N]
  float* __restrict__ hi = p.hin + (b * K * p.dim + c) * p.N + n;
  const int64_t ss = p.dim, hs = p.dim * p.N;
  float am = 1.f, bm = 0.f;   // this lane's map, identity when it holds no chunk
  for (int k = k_lo; k < k_hi; ++k) {
    const float ak = exp2_hw(a2 * S[k * ss]);
    bm = __builtin_fmaf(ak, bm, he[k * hs]);
    am *= ak;
  }
  // inclusive scan over the lanes: the maps of earlier lanes act first
  for (int off = 1; off < kWave; off <<= 1) {
    const float ap = __shfl_up(am, off), bp = __shfl_up(bm, off);
    if (lane >= off) {
      bm = __builtin_fmaf(am, bp, bm);
      am *= ap;
    }
  }
  float ae = __shfl_up(am, 1), be = __shfl_up(bm, 1);
  if (lane == 0) {
    ae = 1.f;
    be = 0.f;
  }
  float h = __builtin_fmaf(ae, he[0], be);   // state entering chunk k_lo
  for (int k = k_lo; k < k_hi; ++k) {
    hi[k * hs] = h;
    h = __builtin_fmaf(exp2_hw(a2 * S[k * ss]), h, he[k * hs]);
  }
  if (p.final_state != nullptr && k_lo < K && k_hi == K) p.final_state[(b * p.dim + c) * p.N + n] = h;
}

// The same carry for few chunks, one lane per (b, c, n) walking the chunks in order: with K - 1 <= 16 the
// wave-level scan would leave most lanes of its waves idle.
__global__ __launch_bounds__(256) void carry_serial_kernel(KernelParams p) {
  const int64_t col = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (col >= p.batch * p.dim * p.N) return;
  const int64_t n = col % p.N;
  const int64_t c = (col / p.N) % p.dim;
  const int64_t b = col / (p.N * p.dim);
  const float a2 = p.A[c * p.N + n] * kLog2e;
  const int K = p.K;
  const float* __restrict__ S = p.S + b * K * p.dim + c;
  const float* __restrict__ he = p.hend + (b * K * p.dim + c) * p.N + n;
  float* __restrict__ hi = p.hin + (b * K * p.dim + c) * p.N + n;
  const int64_t ss = p.dim, hs = p.dim * p.N;
  float h = he[0];   // chunk 0 starts from the true state: its end state enters chunk 1
  for (int k = 1; k < K; ++k) {
    hi[k * hs] = h;
    h = __builtin_fmaf(exp2_hw(a2 * S[k * ss]), h, he[k * hs]);
  }
  if (p.final_state != nullptr) p.final_state[(b * p.dim + c) * p.N + n] = h;
}

// blocks of the carry kernel: one wave per (b, c, n), 4 waves per block
int64_t carry_blocks(int64_t batch, int64_t dim, int64_t N) { return (batch * dim * N + 3) / 4; }

// the carry of a split: few chunks one lane per (b, c, n), else one wave per (b, c, n)
hipError_t launch_carry(const KernelParams& kp, int64_t batch, hipStream_t stream) {
  if (kp.K - 1 <= 16) {
    const int64_t cols = batch * kp.dim * kp.N;
    hipLaunchKernelGGL(carry_serial_kernel, dim3(static_cast<unsigned>((cols + 255) / 256)), dim3(256), 0, stream, kp);
  } else {
    hipLaunchKernelGGL(carry_kernel, dim3(static_cast<unsigned>(carry_blocks(batch, kp.dim, kp.N))), dim3(256), 0,
                       stream, kp);
  }
  return hipGetLastError();
}

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

template <int IO, int G, int NPL, bool VEC, bool FAST>
hipError_t launch_cfg(const KernelParams& kp, int64_t batch, hipStream_t stream) {
  const dim3 block(kThreads);
  if (kp.K == 1) {
    const dim3 grid(static_cast<unsigned>(batch * kp.ngroups));
    hipLaunchKernelGGL((scan_kernel<IO, G, NPL, VEC, FAST, kSingle>), grid, block, 0, stream, kp);
    return hipGetLastError();
  }
  {
    const dim3 grid(static_cast<unsigned>(batch * kp.K * kp.ngroups));
    hipLaunchKernelGGL((scan_kernel<IO, G, NPL, VEC, FAST, kChunk>), grid, block, 0, stream, kp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    hipError_t e = launch_carry(kp, batch, stream);
    if (e != hipSuccess) return e;
  }
  {
    KernelParams kf = kp;
    kf.chunk_offset = 1;
    const dim3 grid(static_cast<unsigned>(batch * (kp.K - 1) * kp.ngroups));
    hipLaunchKernelGGL((scan_kernel<IO, G, NPL, VEC, FAST, kFixup>), grid, block, 0, stream, kf);
    return hipGetLastError();
  }
}

// the same three launches for the one-state-per-lane kernel
template <int IO, int VAR>
hipError_t launch_wide(const KernelParams& kp, int64_t batch, hipStream_t stream) {
  const dim3 block(kThreads);
  if (kp.K == 1) {
    const dim3 grid(static_cast<unsigned>(batch * kp.ngroups));
    hipLaunchKernelGGL((wide_kernel<IO, kSingle, VAR>), grid, block, 0, stream, kp);
    return hipGetLastError();
  }
  {
    const dim3 grid(static_cast<unsigned>(batch * kp.K * kp.ngroups));
    hipLaunchKernelGGL((wide_kernel<IO, kChunk, VAR>), grid, block, 0, stream, kp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    hipError_t e = launch_carry(kp, batch, stream);
    if (e != hipSuccess) return e;
  }
  {
    KernelParams kf = kp;
    kf.chunk_offset = 1;
    const dim3 grid(static_cast<unsigned>(batch * (kp.K - 1) * kp.ngroups));
    hipLaunchKernelGGL((wide_kernel<IO, kFixup, VAR>), grid, block, 0, stream, kf);
    return hipGetLastError();
  }
}

// the same three launches for the one-channel-per-lane kernel: a wave per 64 channels, wpb(IO) waves a workgroup
template <int IO>
hipError_t launch_lane(const KernelParams& kp0, int64_t batch, hipStream_t stream) {
  KernelParams kp = kp0;
  kp.ngroups = static_cast<int>((kp.dim + kWave - 1) / kWave);
  constexpr int WPB = lanek::wpb(IO);
  const dim3 block(kWave * WPB);
  auto blocks = [](int64_t units) { return dim3(static_cast<unsigned>((units + WPB - 1) / WPB)); };
  if (kp.K == 1) {
    hipLaunchKernelGGL((lane_kernel<IO, kSingle>), blocks(batch * kp.ngroups), block, 0, stream, kp);
    return hipGetLastError();
  }
  {
    hipLaunchKernelGGL((lane_kernel<IO, kChunk>), blocks(batch * kp.K * kp.ngroups), block, 0, stream, kp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    hipError_t e = launch_carry(kp, batch, stream);
    if (e != hipSuccess) return e;
  }
  {
    KernelParams kf = kp;
    kf.chunk_offset = 1;
    hipLaunchKernelGGL((lane_kernel<IO, kFixup>), blocks(batch * (kp.K - 1) * kp.ngroups), block, 0, stream, kf);
    return hipGetLastError();
  }
}

template <int IO, int G, int NPL, bool FAST>
hipError_t launch_vec(const KernelParams& kp, bool vec, int64_t batch, hipStream_t stream) {
  if constexpr (Geometry<IO, G, NPL, true, FAST>::VEC_OK) {
    if (vec) return launch_cfg<IO, G, NPL, true, FAST>(kp, batch, stream);
  }
  return launch_cfg<IO, G, NPL, false, FAST>(kp, batch, stream);
}

template <int IO, int G>
hipError_t launch_generic(const KernelParams& kp, int npl, bool vec, int64_t batch, hipStream_t stream) {
  switch (npl) {
    case 4: return launch_vec<IO, G, 4, false>(kp, vec, batch, stream);
    case 8: return launch_vec<IO, G, 8, false>(kp, vec, batch, stream);
    default: return launch_vec<IO, G, 16, false>(kp, vec, batch, stream);
  }
}

template <int IO>
hipError_t launch_io(const KernelParams& kp, int G, int npl, bool vec, int64_t batch, hipStream_t stream) {
  if (kp.conv_w != nullptr || kp.ckpt != nullptr) {   // only in the one-state-per-lane kernel
    if (!(G == 16 && kp.N == 16 && vec)) return hipErrorInvalidValue;
    if (kp.conv_w != nullptr && kp.ckpt != nullptr) return hipErrorInvalidValue;   // not combined
    if (kp.conv_w != nullptr) return launch_wide<IO, kConv>(kp, batch, stream);
    return launch_wide<IO, kCkpt>(kp, batch, stream);
  }
  if (G == 16 && kp.N == 16 && vec) return launch_wide<IO, kPlain>(kp, batch, stream);
  if (kp.N <= 16) {
    switch (G) {
      case 1:
        if (kp.N == 16 && vec) return launch_lane<IO>(kp, batch, stream);
        return launch_vec<IO, 1, 16, true>(kp, vec, batch, stream);
      case 2: return launch_vec<IO, 2, 8, true>(kp, vec, batch, stream);
      case 4: return launch_vec<IO, 4, 4, true>(kp, vec, batch, stream);
      case 8: return launch_vec<IO, 8, 4, false>(kp, vec, batch, stream);
      default: return launch_vec<IO, 16, 4, false>(kp, vec, batch, stream);
    }
  }
  switch (G) {
    case 2: return launch_vec<IO, 2, 16, false>(kp, vec, batch, stream);
    case 4: return launch_generic<IO, 4>(kp, npl < 8 ? 8 : npl, vec, batch, stream);
    case 8: return launch_generic<IO, 8>(kp, npl, vec, batch, stream);
    default: return launch_generic<IO, 16>(kp, npl, vec, batch, stream);
  }
}

int states_per_lane(int G, int64_t N) {
  const int64_t need = (N + G - 1) / G;
  return need <= 4 ? 4 : (need <= 8 ? 8 : 16);
}

}  // namespace

size_t scan_checkpoint_bytes(int64_t batch, int64_t L, int64_t dim) {
  return static_cast<size_t>(batch) * static_cast<size_t>((L + 15) / 16) * static_cast<size_t>((dim + 15) / 16 * 16) *
         16 * sizeof(float);
}

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
  kp.conv_w = a.conv_w; kp.conv_b = a.conv_b; kp.conv_init = a.conv_init; kp.conv_width = a.conv_width;
  kp.batch = a.batch; kp.L = a.L; kp.dim = a.dim; kp.N = a.N;
  kp.K = a.K;
  kp.chunk_len = (a.L + a.K - 1) / a.K;
  kp.ckpt = a.ckpt;
  kp.ckpt_tiles = (a.L + 15) / 16;
  if (a.ckpt != nullptr) {   // chunks start on checkpoint tiles (the plan's K is an upper bound)
    kp.chunk_len = (kp.chunk_len + 15) / 16 * 16;
    kp.K = a.L > 0 ? static_cast<int>((a.L + kp.chunk_len - 1) / kp.chunk_len) : 1;
  }
  kp.chunk_offset = 0;
  const int G = a.G;
  const int cpb = kThreads / G;
  kp.ngroups = static_cast<int>((a.dim + cpb - 1) / cpb);
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
  const int64_t es = a.io == 1 ? 2 : 4;
  auto al16 = [](const void* q) { return q == nullptr || (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  // 16-byte B/C loads need N / (elements per 16 bytes) to be a power of two
  const int64_t bc_chunks = (a.N * es) / 16;
  const bool bc_pow2 = (a.N * es) % 16 == 0 && bc_chunks > 0 && (bc_chunks & (bc_chunks - 1)) == 0;
  kp.bc_shift = 0;
  while (bc_pow2 && (int64_t{1} << kp.bc_shift) < bc_chunks) ++kp.bc_shift;
  const bool vec = (a.dim * es) % 16 == 0 && bc_pow2 && al16(a.x) && al16(a.delta) && al16(a.z) &&
                   al16(a.B) && al16(a.C) && al16(a.out) && al16(a.conv_init);
  if (a.io == 1) return launch_io<1>(kp, G, npl, vec, a.batch, stream);
  return launch_io<0>(kp, G, npl, vec, a.batch, stream);
}

}  // namespace mssm
