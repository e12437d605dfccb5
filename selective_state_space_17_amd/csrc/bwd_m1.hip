// Gradients of the Mamba-1 selective scan for gfx950 (MI355X).
//
// The forward operation is the selective recurrence of "P20 - Mamba", 5 and
// "03 - Modelos de espacio de estados" ("El mecanismo selectivo de Mamba",
// "Discretizacion"): per (b, c, n) and time t
//   a_t = exp(delta_t A[c,n]),  h_t = a_t h_{t-1} + delta_t B_t[n] x_t,
//   y_t = sum_n C_t[n] h_t + D[c] x_t,  out_t = y_t silu(z_t).
// Reverse mode through that loop, for upstream gradients g_t = dL/dout_t and
// dL/dh_{L-1} (dfinal):
//   dy_t = g_t silu(z_t),  dz_t = g_t y_t silu'(z_t)
//   lam_t = C_t dy_t + a_{t+1} lam_{t+1}         (adjoint of h_t)
//   dC_t[n] = sum_c dy_t h_t,   dB_t[n] = sum_c lam_t delta_t x_t
//   ddelta_t = sum_n lam_t (A a_t h_{t-1}) + x_t sum_n lam_t B_t
//   dx_t = D dy_t + delta_t sum_n lam_t B_t
//   dA[c,n] = sum_{b,t} lam_t a_t h_{t-1} delta_t,  dD[c] = sum_{b,t} dy_t x_t
//   dh0 = a_0 lam_0
//
// Mapping.  A block of 4 waves owns 16 channels of one batch row and one
// slice of 16 states; lane (row cl = tid/16, n = tid%16) holds state
// 16 * slice + n of channel c0 + cl (states past dstate carry zeros).  The
// slices of a channel are independent except in the three sums over all
// states (y for dz, and the two sums that make ddelta and dx): with more than
// one slice each block writes its partial sums, and a finishing kernel adds
// them in slice order and forms dz, ddelta and dx.  The reverse walk needs
// h_{t-1} at every step, so:
//   phase A  walks the sequence forward once (the exp and FMA of the
//            forward recurrence only) and writes the state entering every
//            16-step tile to a checkpoint workspace;
//   phase B  walks the tiles backwards; per tile it reloads the checkpoint,
//            recomputes the 16 states and decays into registers, then runs
//            the adjoint recursion over them.
// Per-(t, c) values (delta, delta*x, dy) and per-(t, n) values (B, C) are
// staged in LDS once per tile.  Sums over the 16 states of a channel (y for
// dz, and the two sums that make ddelta and dx) are done by writing each
// lane's 16 per-step products to LDS and reading them back transposed, so
// lane (cl, s) adds the 16 products of step s; sums over the 16 channels of
// a block (dB, dC) go through the same LDS area and are written as one
// partial per block, which a second kernel adds in a fixed order (the result
// does not depend on scheduling).  dA and dD partials per batch row are
// added the same way.
#include "internal.h"

namespace mssm {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kThreads = 256;
constexpr int kCPB = 16;   // channels per block
constexpr int kTT = 16;    // steps per tile (= checkpoint interval)

template <typename T> struct Io;
template <> struct Io<float> {
  __device__ static float raw(const void* p, int64_t i) { return static_cast<const float*>(p)[i]; }
  __device__ static float cvt(float v) { return v; }
  __device__ static float get(const void* p, int64_t i) { return static_cast<const float*>(p)[i]; }
  __device__ static void put(void* p, int64_t i, float v) { static_cast<float*>(p)[i] = v; }
};
template <> struct Io<uint16_t> {
  __device__ static uint16_t raw(const void* p, int64_t i) { return static_cast<const uint16_t*>(p)[i]; }
  __device__ static float cvt(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
  __device__ static float get(const void* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
  }
  __device__ static void put(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));   // nearest even
  }
};

__device__ __forceinline__ float exp2_hw(float v) { return __builtin_amdgcn_exp2f(v); }

template <int CTRL> __device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
// with bound_ctrl set, for controls whose every source lane exists (a row rotation), so that the
// compiler folds the move into the consuming add
template <int CTRL> __device__ __forceinline__ float dpp_bc(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
// sum over the 16 lanes of a row, result in every lane
__device__ __forceinline__ float row_sum(float v) {
  v += dpp<0x128>(v);   // row_ror:8
  v += dpp<0x124>(v);   // row_ror:4
  v += dpp<0x122>(v);   // row_ror:2
  v += dpp<0x121>(v);   // row_ror:1
  return v;
}

// Transpose areas: 16 rows (channels) x 16 states x 16 steps of fp32, row
// stride 272.  Lane (cl, n) writes its 16 steps as four 16-byte stores at
// qpos(cl, n, 4i); lane (cl, s) reads state n of step s, and a thread of the
// channel sums reads row r.  The LDS serves 32 banks: a 16-byte store per
// 8 lanes, a 4-byte read per 32 lanes.  The row stride (272 = 16 mod 32) and
// the xor of the step by bits 1-2 of the state put each of those groups on
// distinct banks, and the read addresses are affine in the loop index.
constexpr int kRow = 272;
__device__ __forceinline__ int qpos(int cl, int n, int s) { return cl * kRow + 16 * n + (s ^ (((n >> 1) & 3) << 2)); }
constexpr int kBT = 20;   // B^T / C^T row stride: lane n reads 4 steps with one 16-byte load
constexpr int kBA = 68;   // the same for the 64-step staging tiles of the forward walk

template <int S> __device__ __forceinline__ float bcast(float v) { return dpp<0x150 + S>(v); }   // row_newbcast:S

// acc += bcast<S>(b) * o as one v_fmac_f32_dpp (the compiler does not fold a
// DPP operand into an FMA that accumulates in place).  b must not have been
// written by the two preceding VALU instructions (it is written once per tile).
template <int S> __device__ __forceinline__ void fmac_bcast(float& acc, float b, float o);
#define MSSM_FMAC_BCAST(S)                                                                              \
  template <> __device__ __forceinline__ void fmac_bcast<S>(float& acc, float b, float o) {            \
    asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:" #S " row_mask:0xf bank_mask:0xf"             \
                 : "+v"(acc) : "v"(b), "v"(o));                                                        \
  }
MSSM_FMAC_BCAST(0) MSSM_FMAC_BCAST(1) MSSM_FMAC_BCAST(2) MSSM_FMAC_BCAST(3)
MSSM_FMAC_BCAST(4) MSSM_FMAC_BCAST(5) MSSM_FMAC_BCAST(6) MSSM_FMAC_BCAST(7)
MSSM_FMAC_BCAST(8) MSSM_FMAC_BCAST(9) MSSM_FMAC_BCAST(10) MSSM_FMAC_BCAST(11)
MSSM_FMAC_BCAST(12) MSSM_FMAC_BCAST(13) MSSM_FMAC_BCAST(14) MSSM_FMAC_BCAST(15)
#undef MSSM_FMAC_BCAST

// bcast<S>(b) * o as one v_mul_f32_dpp, written out where a product is used
// (the compiler would otherwise hoist the 16 broadcasts and keep them in VGPRs)
template <int S> __device__ __forceinline__ float mul_bcast(float b, float o);
#define MSSM_MUL_BCAST(S)                                                                               \
  template <> __device__ __forceinline__ float mul_bcast<S>(float b, float o) {                        \
    float r;                                                                                           \
    asm volatile("v_mul_f32_dpp %0, %1, %2 row_newbcast:" #S " row_mask:0xf bank_mask:0xf"              \
                 : "=v"(r) : "v"(b), "v"(o));                                                          \
    return r;                                                                                          \
  }
MSSM_MUL_BCAST(0) MSSM_MUL_BCAST(1) MSSM_MUL_BCAST(2) MSSM_MUL_BCAST(3)
MSSM_MUL_BCAST(4) MSSM_MUL_BCAST(5) MSSM_MUL_BCAST(6) MSSM_MUL_BCAST(7)
MSSM_MUL_BCAST(8) MSSM_MUL_BCAST(9) MSSM_MUL_BCAST(10) MSSM_MUL_BCAST(11)
MSSM_MUL_BCAST(12) MSSM_MUL_BCAST(13) MSSM_MUL_BCAST(14) MSSM_MUL_BCAST(15)
#undef MSSM_MUL_BCAST

struct BwdParams {
  const void* x;
  const void* delta;
  const void* B;
  const void* C;
  const void* z;       // nullable
  const void* dout;
  const float* A;
  const float* D;      // nullable
  const float* h0;     // nullable
  const float* dfinal; // nullable
  void* dx;
  void* ddelta;
  void* dz;            // written iff z != nullptr
  float* dh0;          // nullable
  float* ckpt;         // [batch][ntiles][ncb*16][np16]
  const float* ckpt_in;   // nullable: the same array written by the training-mode forward (dstate 16)
  float* partB;        // [ncb][batch][L][np16]
  float* partC;        // [ncb][batch][L][np16]
  float* wsA;          // [batch][ncb*16][np16]
  float* wsD;          // [batch][ncb*16]
  float* part_y;       // [nsl][batch][L][dim]: with several slices, each slice's share of
  float* part_s1;      //   sum_n C h, of sum_n lam a h A (ddelta) and of sum_n lam B (ddelta, dx)
  float* part_s2;
  int64_t batch, L, dim, N;
  int ntiles, ncb;
  int nsl, np16;       // state slices of 16, and 16 * nsl
};

// Step S of the forward recurrence for lane (cl, n): the per-(t, c) values
// of step S sit in lane S of the row and reach every lane through a DPP
// row broadcast folded into the multiply.
template <int S>
__device__ __forceinline__ void fwd_step(float& h, float& a, float dl, float du, float A2, float b) {
  a = exp2_hw(bcast<S>(dl) * A2);
  h = __builtin_fmaf(a, h, bcast<S>(du) * b);
}

template <int G>
__device__ __forceinline__ void fwd_group(float& h, float dl, float du, float A2, const float4& b4) {
  float a;
  fwd_step<4 * G + 0>(h, a, dl, du, A2, b4.x);
  fwd_step<4 * G + 1>(h, a, dl, du, A2, b4.y);
  fwd_step<4 * G + 2>(h, a, dl, du, A2, b4.z);
  fwd_step<4 * G + 3>(h, a, dl, du, A2, b4.w);
}

template <int S>
__device__ __forceinline__ void rec_step(float& h, float (&av)[16], float (&hs)[16], float (&pr)[16], float (&q1)[16],
                                         float dl, float du, float dy, float A2, float b, float cc) {
  fwd_step<S>(h, av[S], dl, du, A2, b);
  hs[S] = h;
  pr[S] = cc * h;                // C h: readout term of y
  q1[S] = mul_bcast<S>(dy, h);   // dy h: dC term
}

template <int S>
__device__ __forceinline__ void adj_step(float& lam, float& dA, const float (&av)[16], const float (&hs)[16], float hin,
                                         float (&ls)[16], float (&r1)[16], float dl, float dy, float Av, float cc) {
  fmac_bcast<S>(lam, dy, cc);                     // + C dy: lam_t
  ls[S] = lam;                                    // (lam_t B and lam_t delta x are formed when parked)
  lam *= av[S];                                   // a_t lam_t
  const float t1 = lam * (S > 0 ? hs[S > 0 ? S - 1 : 0] : hin);   // lam a_t h_{t-1}
  fmac_bcast<S>(dA, dl, t1);                      // + lam a_t h_{t-1} delta_t
  r1[S] = t1 * Av;
  // keep this step's results here (otherwise the compiler keeps operands of
  // later-consumed values alive across the loop)
  __asm__ volatile("" : "+v"(ls[S]), "+v"(r1[S]));
}

// three waves per SIMD: what the grid of a typical layer provides (batch x dim / 16 blocks of 4 waves)
// SPLIT: more than one state slice (partial sums out, finished by bwd_finish)
template <typename T, bool SPLIT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void scan_bwd_kernel(BwdParams p) {
  using io = Io<T>;
  __shared__ __attribute__((aligned(16))) float BT[16 * kBT];      // B^T per tile
  __shared__ __attribute__((aligned(16))) float CT[16 * kBT];      // C^T per tile
  __shared__ __attribute__((aligned(16))) float Q1[16 * kRow];     // dy*h (dC) / transposes
  __shared__ __attribute__((aligned(16))) float Q2[16 * kRow];     // lam*delta*x (dB) / transposes

  const int tid = threadIdx.x;
  const int cl = tid >> 4;          // channel row; also: staging / finishing thread of step fs = n
  const int n = tid & 15;           // state
  const int fs = n;
  // block -> (batch row, channel block); blocks are dealt to the 8 XCDs in
  // turn, so consecutive blocks are remapped to put 4 neighbouring channel
  // blocks (one 128-byte line of a bf16 row) on one XCD, whose L2 then serves
  // them all
  // (the slices of one channel block are consecutive blocks)
  const int slice = SPLIT ? static_cast<int>(blockIdx.x % p.nsl) : 0;
  const int64_t nb = SPLIT ? gridDim.x / p.nsl : gridDim.x;
  const int64_t bid = SPLIT ? blockIdx.x / p.nsl : blockIdx.x;
  int64_t lin = bid;
  if (bid < (nb / 32) * 32) {
    const int64_t xcd = bid % 8, rr = bid / 8;
    lin = ((rr / 4) * 8 + xcd) * 4 + rr % 4;
  }
  const int cb = static_cast<int>(lin % p.ncb);
  const int64_t b = lin / p.ncb;
  const int64_t c0 = static_cast<int64_t>(cb) * kCPB;
  const int64_t c = c0 + cl;
  const int64_t L = p.L, dim = p.dim, N = p.N;
  const int s0 = 16 * slice;           // first state of the slice
  const int64_t sn = s0 + n;           // this lane's state
  const bool lane_ok = c < dim && sn < N;
  const int64_t D16 = static_cast<int64_t>(p.ncb) * kCPB;
  const int64_t NP = p.np16;
  const int bs = tid >> 4, bn = tid & 15;   // B/C staging: step, state s0 + bn

  const float Av = lane_ok ? p.A[c * N + sn] : 0.f;
  const float A2 = Av * kLog2e;
  float* ck = p.ckpt + (b * p.ntiles * D16 + c) * NP + sn;   // + k * D16 * NP
  // the checkpoints phase B starts its tiles from: the forward's, or phase A's
  const float* ckr = p.ckpt_in != nullptr ? p.ckpt_in + (b * p.ntiles * D16 + c) * NP + sn : ck;

  // -------------------------------------------------------------- phase A
  // Staged 64 steps at a time (one barrier per 64 steps, loads a whole
  // staging tile ahead); the state entering every 16-step tile is stored.
  // Skipped when the training-mode forward already stored them.
  if (p.ckpt_in == nullptr) {
    float* BA = Q1;   // B^T of a 64-step staging tile: [2 buffers][16 states][kBA]
    float h = (lane_ok && p.h0 != nullptr) ? p.h0[(b * dim + c) * N + sn] : 0.f;
    // Loads are unconditional, from an in-range element when the step or
    // channel is past the end, and their raw values are left untouched until
    // the tile is staged (masking or widening them at once would make the
    // wave wait for the load there instead of a tile later).
    T rd[4], rx[4], rb[4];
    bool ok[4], okb[4];
    auto issue = [&](int64_t t0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t t = t0 + 16 * j + fs;
        ok[j] = t < L && c < dim;
        const int64_t i = (b * L + (t < L ? t : L - 1)) * dim + (c < dim ? c : dim - 1);
        rd[j] = io::raw(p.delta, i);
        rx[j] = io::raw(p.x, i);
        const int64_t tb = t0 + 16 * j + bs;
        okb[j] = tb < L && s0 + bn < N;
        rb[j] = io::raw(p.B, (b * L + (tb < L ? tb : L - 1)) * N + (s0 + bn < N ? s0 + bn : N - 1));
      }
    };
    // tiles 0 .. ntiles-2 are walked (their end states are checkpoints 1 .. ntiles-1)
    const int64_t walk = static_cast<int64_t>(p.ntiles - 1) * kTT;
    if (walk > 0) issue(0);
    int buf = 0;
    for (int64_t t0 = 0; t0 < walk; t0 += 64, buf ^= 1) {
      float* ba = BA + buf * 16 * kBA;
      float dl[4], du[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ba[bn * kBA + 16 * j + bs] = okb[j] ? io::cvt(rb[j]) : 0.f;
        dl[j] = ok[j] ? io::cvt(rd[j]) : 0.f;
        du[j] = dl[j] * (ok[j] ? io::cvt(rx[j]) : 0.f);
      }
      __syncthreads();
      if (t0 + 64 < walk) issue(t0 + 64);
      const float4* b4 = reinterpret_cast<const float4*>(ba + n * kBA);
      const int k0 = static_cast<int>(t0 / kTT);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (t0 + 16 * j < walk) {   // uniform
          ck[static_cast<int64_t>(k0 + j) * D16 * NP] = h;   // padded lanes store their zero state too
          fwd_group<0>(h, dl[j], du[j], A2, b4[4 * j + 0]);
          fwd_group<1>(h, dl[j], du[j], A2, b4[4 * j + 1]);
          fwd_group<2>(h, dl[j], du[j], A2, b4[4 * j + 2]);
          fwd_group<3>(h, dl[j], du[j], A2, b4[4 * j + 3]);
        }
      }
    }
    if (p.ntiles > 0) ck[static_cast<int64_t>(p.ntiles - 1) * D16 * NP] = h;
    __syncthreads();   // orders the checkpoint stores before phase B's loads; frees Q1
  }

  // -------------------------------------------------------------- phase B
  const float Dc = (c < dim && p.D != nullptr) ? p.D[c] : 0.f;
  float lam = (lane_ok && p.dfinal != nullptr) ? p.dfinal[(b * dim + c) * N + sn] : 0.f;
  float dAacc = 0.f, dDacc = 0.f;
  // raw prefetched values of the next tile (unconditional in-range loads, see phase A)
  T rdl{}, rx{}, rg{}, rz{}, rb{}, rc{};
  float rh = 0.f;
  bool ok = false, okb = false;
  auto issue = [&](int k) {
    const int64_t t = static_cast<int64_t>(k) * kTT + fs;
    ok = t < L && c < dim;
    const int64_t i = (b * L + (t < L ? t : L - 1)) * dim + (c < dim ? c : dim - 1);
    rdl = io::raw(p.delta, i);
    rx = io::raw(p.x, i);
    rg = io::raw(p.dout, i);
    if (p.z != nullptr) rz = io::raw(p.z, i);
    const int64_t tb = static_cast<int64_t>(k) * kTT + bs;
    okb = tb < L && s0 + bn < N;
    const int64_t ib = (b * L + (tb < L ? tb : L - 1)) * N + (s0 + bn < N ? s0 + bn : N - 1);
    rb = io::raw(p.B, ib);
    rc = io::raw(p.C, ib);
    rh = ckr[static_cast<int64_t>(k) * D16 * NP];   // channels past dim: masked at staging
  };
  // transposes through this wave's own rows of Q1/Q2 (no other wave touches
  // them before the barrier that ends the tile's compute); a wave's LDS
  // accesses run in order, so a row is rewritten only after the reads issued
  // before the rewrite have been served
  auto park = [&](float* area, const float (&v)[kTT]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<float4*>(&area[qpos(cl, n, 4 * i)]) = float4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
    __builtin_amdgcn_wave_barrier();
  };
  // Sums over the 16 states: lanes n and n+8 first add their 16 per-step
  // products with a DPP row rotation (half the bytes through LDS); lanes 0-7
  // park those pair sums, and lane (cl, fs) reads the 8 of step fs (the sum is
  // taken later, so other work can cover the LDS latency)
  auto park_pairs = [&](float* area, const float (&v)[kTT]) {
    float ps[kTT];
    {
#pragma clang fp contract(off)   // an FMA with the product would leave the DPP move unfolded
#pragma unroll
      for (int i = 0; i < kTT; ++i) ps[i] = v[i] + dpp_bc<0x128>(v[i]);   // row_ror:8
    }
    asm volatile("" : "+v"(ps[0]), "+v"(ps[1]), "+v"(ps[2]), "+v"(ps[3]), "+v"(ps[4]), "+v"(ps[5]), "+v"(ps[6]),
                 "+v"(ps[7]));
    asm volatile("" : "+v"(ps[8]), "+v"(ps[9]), "+v"(ps[10]), "+v"(ps[11]), "+v"(ps[12]), "+v"(ps[13]),
                 "+v"(ps[14]), "+v"(ps[15]));
    if (n < 8) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<float4*>(&area[qpos(cl, n, 4 * i)]) = float4{ps[4 * i], ps[4 * i + 1], ps[4 * i + 2], ps[4 * i + 3]};
    }
    __builtin_amdgcn_wave_barrier();
  };
  auto fetch = [&](const float* area, float (&r)[8]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {   // pair sums of states 2m, 2m + 1
      const float* base = area + cl * kRow + 32 * m + (fs ^ ((m & 3) << 2));
      r[2 * m] = base[0];
      r[2 * m + 1] = base[16];
    }
  };
  auto sum8 = [](const float (&r)[8]) { return ((r[0] + r[1]) + (r[2] + r[3])) + ((r[4] + r[5]) + (r[6] + r[7])); };

  if (p.ntiles > 0) issue(p.ntiles - 1);
  for (int k = p.ntiles - 1; k >= 0; --k) {
    const int64_t t0 = static_cast<int64_t>(k) * kTT;
    const int64_t tf = t0 + fs;
    const bool fvalid = tf < L && c < dim;
    // ---- stage: step fs of channel cl stays in this thread's registers, the
    // source of the row broadcasts and of the finish
    const float dl = ok ? io::cvt(rdl) : 0.f, u = ok ? io::cvt(rx) : 0.f, du = dl * u;
    const float g = ok ? io::cvt(rg) : 0.f;
    float dy = g, sdz = 0.f;
    if (p.z != nullptr) {
      const float zz = io::cvt(rz);
      const float sg = __builtin_amdgcn_rcpf(1.f + exp2_hw(-zz * kLog2e));
      dy = g * zz * sg;
      sdz = g * sg * __builtin_fmaf(zz, 1.f - sg, 1.f);
    }
    BT[bn * kBT + bs] = okb ? io::cvt(rb) : 0.f;
    CT[bn * kBT + bs] = okb ? io::cvt(rc) : 0.f;
    const float hin = c < dim ? rh : 0.f;   // state entering the tile (rh is reloaded below)
    float h = hin;
    __syncthreads();
    if (k > 0) issue(k - 1);
    const float4* b4 = reinterpret_cast<const float4*>(&BT[n * kBT]);
    const float4* c4 = reinterpret_cast<const float4*>(&CT[n * kBT]);

    // ---- recompute the tile's states and decays
    float hs[kTT], av[kTT], pr[kTT], q1[kTT];
    {
      float4 bv = b4[0], cv = c4[0];
      rec_step<0>(h, av, hs, pr, q1, dl, du, dy, A2, bv.x, cv.x);
      rec_step<1>(h, av, hs, pr, q1, dl, du, dy, A2, bv.y, cv.y);
      rec_step<2>(h, av, hs, pr, q1, dl, du, dy, A2, bv.z, cv.z);
      rec_step<3>(h, av, hs, pr, q1, dl, du, dy, A2, bv.w, cv.w);
      bv = b4[1]; cv = c4[1];
      rec_step<4>(h, av, hs, pr, q1, dl, du, dy, A2, bv.x, cv.x);
      rec_step<5>(h, av, hs, pr, q1, dl, du, dy, A2, bv.y, cv.y);
      rec_step<6>(h, av, hs, pr, q1, dl, du, dy, A2, bv.z, cv.z);
      rec_step<7>(h, av, hs, pr, q1, dl, du, dy, A2, bv.w, cv.w);
      bv = b4[2]; cv = c4[2];
      rec_step<8>(h, av, hs, pr, q1, dl, du, dy, A2, bv.x, cv.x);
      rec_step<9>(h, av, hs, pr, q1, dl, du, dy, A2, bv.y, cv.y);
      rec_step<10>(h, av, hs, pr, q1, dl, du, dy, A2, bv.z, cv.z);
      rec_step<11>(h, av, hs, pr, q1, dl, du, dy, A2, bv.w, cv.w);
      bv = b4[3]; cv = c4[3];
      rec_step<12>(h, av, hs, pr, q1, dl, du, dy, A2, bv.x, cv.x);
      rec_step<13>(h, av, hs, pr, q1, dl, du, dy, A2, bv.y, cv.y);
      rec_step<14>(h, av, hs, pr, q1, dl, du, dy, A2, bv.z, cv.z);
      rec_step<15>(h, av, hs, pr, q1, dl, du, dy, A2, bv.w, cv.w);
    }
    park_pairs(Q2, pr);
    float ry[8];
    fetch(Q2, ry);           // y of step fs, summed after the adjoint loop
    const int64_t fi = (b * L + tf) * dim + c;

    // ---- adjoint recursion over the tile, last step first
    float ls[kTT], r1[kTT];
    {
      __asm__ volatile("" ::: "memory");   // B, C are read again here, not kept from the loop above
      __asm__ volatile("s_nop 1");   // DPP reads of dl / dy below: their last VALU write is long past
      float4 cv = c4[3];
      adj_step<15>(lam, dAacc, av, hs, hin, ls, r1, dl, dy, Av, cv.w);
      adj_step<14>(lam, dAacc, av, hs, hin, ls, r1, dl, dy, Av, cv.z);
      adj_step<13>(lam, dAacc, av, hs, hin, ls, r1, dl, dy, Av, cv.y);
      adj_step<12>(lam, dAacc, av, hs, hin, ls, r1, dl, dy, Av, cv.x);
      cv = c4[2];
      adj_step<11>(lam, dAacc, av, hs, hin, ls, r1, dl, dy, Av, cv.w);
      adj_step<10>(lam, dAacc, av, hs, hin, ls, r1, dl, dy, Av, cv.z);
      adj_step<9>(lam, dAacc, av, hs, hin, ls, r1, dl, dy, Av, cv.y);
      adj_step<8>(lam, dAacc, av, hs, hin, ls, r1, dl, dy, Av, cv.x);
      cv = c4[1];
      adj_step<7>(lam, dAacc, av, hs, hin, ls, r1, dl, dy, Av, cv.w);
      adj_step<6>(lam, dAacc, av, hs, hin, ls, r1, dl, dy, Av, cv.z);
      adj_step<5>(lam, dAacc, av, hs, hin, ls, r1, dl, dy, Av, cv.y);
      adj_step<4>(lam, dAacc, av, hs, hin, ls, r1, dl, dy, Av, cv.x);
      cv = c4[0];
      adj_step<3>(lam, dAacc, av, hs, hin, ls, r1, dl, dy, Av, cv.w);
      adj_step<2>(lam, dAacc, av, hs, hin, ls, r1, dl, dy, Av, cv.z);
      adj_step<1>(lam, dAacc, av, hs, hin, ls, r1, dl, dy, Av, cv.y);
      adj_step<0>(lam, dAacc, av, hs, hin, ls, r1, dl, dy, Av, cv.x);
    }
    const float yp = sum8(ry);   // this slice's sum_n C h
    if constexpr (!SPLIT) {
      if (p.z != nullptr && fvalid) io::put(p.dz, fi, sdz * __builtin_fmaf(Dc, u, yp));
    }
    // both sums over states in one LDS round trip (Q1's rows take q1 after)
    park_pairs(Q1, r1);
    {
      float r2[kTT];   // lam_t B_t
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 bv = b4[g];
        r2[4 * g] = ls[4 * g] * bv.x;
        r2[4 * g + 1] = ls[4 * g + 1] * bv.y;
        r2[4 * g + 2] = ls[4 * g + 2] * bv.z;
        r2[4 * g + 3] = ls[4 * g + 3] * bv.w;
      }
      park_pairs(Q2, r2);
    }
    float ra[8], rb2[8];
    fetch(Q1, ra);
    fetch(Q2, rb2);
    dDacc = __builtin_fmaf(dy, u, dDacc);
    const float s1 = sum8(ra), s2 = sum8(rb2);
    if (fvalid) {
      if constexpr (SPLIT) {
        const int64_t pi = ((static_cast<int64_t>(slice) * p.batch + b) * L + tf) * dim + c;
        p.part_y[pi] = yp;
        p.part_s1[pi] = s1;
        p.part_s2[pi] = s2;
      } else {
        io::put(p.ddelta, fi, __builtin_fmaf(u, s2, s1));
        io::put(p.dx, fi, __builtin_fmaf(dl, s2, Dc * dy));
      }
    }
    park(Q1, q1);
    {
      float q2[kTT];   // lam_t delta_t x_t
      q2[0] = mul_bcast<0>(du, ls[0]);     q2[1] = mul_bcast<1>(du, ls[1]);     q2[2] = mul_bcast<2>(du, ls[2]);
      q2[3] = mul_bcast<3>(du, ls[3]);     q2[4] = mul_bcast<4>(du, ls[4]);     q2[5] = mul_bcast<5>(du, ls[5]);
      q2[6] = mul_bcast<6>(du, ls[6]);     q2[7] = mul_bcast<7>(du, ls[7]);     q2[8] = mul_bcast<8>(du, ls[8]);
      q2[9] = mul_bcast<9>(du, ls[9]);     q2[10] = mul_bcast<10>(du, ls[10]); q2[11] = mul_bcast<11>(du, ls[11]);
      q2[12] = mul_bcast<12>(du, ls[12]); q2[13] = mul_bcast<13>(du, ls[13]); q2[14] = mul_bcast<14>(du, ls[14]);
      q2[15] = mul_bcast<15>(du, ls[15]);
      park(Q2, q2);
    }
    __syncthreads();

    // ---- channel sums of this block: thread (step rs, state rn); each half
    // wave takes 4 steps x 8 states, which the layout spreads over 32 banks
    {
      float sb = 0.f, sc = 0.f;
      const int rn = (tid & 7) | (((tid >> 5) & 1) << 3);
      const int rs = ((tid >> 3) & 3) | ((tid >> 6) << 2);
      const int base = qpos(0, rn, rs);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sc += Q1[base + r * kRow];
        sb += Q2[base + r * kRow];
      }
      const int64_t t = t0 + rs;
      if (t < L) {
        const int64_t o = ((static_cast<int64_t>(cb) * p.batch + b) * L + t) * NP + s0 + rn;
        p.partB[o] = sb;
        p.partC[o] = sc;
      }
    }
    // No barrier here: B^T / C^T are not read after the one above, so the next
    // tile may stage them at once, and Q1 / Q2 are written again only after
    // the next tile's first barrier, which every wave reaches after its sums.
  }

  if (lane_ok && p.dh0 != nullptr) p.dh0[(b * dim + c) * N + sn] = lam;
  p.wsA[(b * D16 + c) * NP + sn] = dAacc;   // zero for padded lanes
  const float dDrow = row_sum(dDacc);     // the same in every slice: slice 0 stores it
  if (n == 0 && slice == 0) p.wsD[b * D16 + c] = dDrow;
}

// With several state slices: y = sum of the slices' shares + D x, and the two
// state sums, added in slice order, then dz, ddelta and dx as the gradient
// kernel forms them with one slice.
template <typename T>
__global__ __launch_bounds__(256) void bwd_finish(BwdParams p) {
  using io = Io<T>;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // (b, t, c)
  const int64_t n_bld = p.batch * p.L * p.dim;
  if (i >= n_bld) return;
  const int64_t c = i % p.dim;
  float yp = 0.f, s1 = 0.f, s2 = 0.f;
  for (int sl = 0; sl < p.nsl; ++sl) {
    yp += p.part_y[sl * n_bld + i];
    s1 += p.part_s1[sl * n_bld + i];
    s2 += p.part_s2[sl * n_bld + i];
  }
  const float dl = io::get(p.delta, i), u = io::get(p.x, i), g = io::get(p.dout, i);
  const float Dc = p.D != nullptr ? p.D[c] : 0.f;
  float dy = g;
  if (p.z != nullptr) {
    const float zz = io::get(p.z, i);
    const float sg = __builtin_amdgcn_rcpf(1.f + exp2_hw(-zz * kLog2e));
    dy = g * zz * sg;
    io::put(p.dz, i, g * sg * __builtin_fmaf(zz, 1.f - sg, 1.f) * __builtin_fmaf(Dc, u, yp));
  }
  io::put(p.ddelta, i, __builtin_fmaf(u, s2, s1));
  io::put(p.dx, i, __builtin_fmaf(dl, s2, Dc * dy));
}

// dB, dC: sum of the per-block partials, in block order.  A thread owns four
// consecutive (step, state) slots (16-byte loads) and keeps several blocks'
// loads in flight; the order of the additions is fixed.
__global__ __launch_bounds__(256) void bwd_reduce_bc(const float* partB, const float* partC, float* dB, float* dC,
                                                     int64_t batch, int64_t L, int64_t N, int ncb, int np16) {
  const int64_t rows = batch * L;
  const int64_t g4 = np16 / 4;   // 4-state groups per row
  const int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // (row, 4-state group)
  if (q >= rows * g4) return;
  const int64_t stride = rows * g4;   // float4 slots per block's partial
  const float4* pb = reinterpret_cast<const float4*>(partB) + q;
  const float4* pc = reinterpret_cast<const float4*>(partC) + q;
  float4 sb = {0.f, 0.f, 0.f, 0.f}, sc = {0.f, 0.f, 0.f, 0.f};
  int k = 0;
  for (; k + 4 <= ncb; k += 4) {
    float4 vb[4], vc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vb[j] = pb[(k + j) * stride];
      vc[j] = pc[(k + j) * stride];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sb.x += vb[j].x; sb.y += vb[j].y; sb.z += vb[j].z; sb.w += vb[j].w;
      sc.x += vc[j].x; sc.y += vc[j].y; sc.z += vc[j].z; sc.w += vc[j].w;
    }
  }
  for (; k < ncb; ++k) {
    const float4 vb = pb[k * stride], vc = pc[k * stride];
    sb.x += vb.x; sb.y += vb.y; sb.z += vb.z; sb.w += vb.w;
    sc.x += vc.x; sc.y += vc.y; sc.z += vc.z; sc.w += vc.w;
  }
  const int64_t row = q / g4;
  const int n0 = static_cast<int>(q % g4) * 4;
  const float b4[4] = {sb.x, sb.y, sb.z, sb.w}, c4[4] = {sc.x, sc.y, sc.z, sc.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (n0 + j < N) {
      dB[row * N + n0 + j] = b4[j];
      dC[row * N + n0 + j] = c4[j];
    }
  }
}

// dA, dD: sum over the batch rows, in order
__global__ __launch_bounds__(256) void bwd_reduce_ad(const float* wsA, const float* wsD, float* dA, float* dD,
                                                     int64_t batch, int64_t dim, int64_t N, int ncb, int np16) {
  const int64_t D16 = static_cast<int64_t>(ncb) * 16;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // (c, padded state)
  if (i >= dim * np16) return;
  const int64_t cc = i / np16;
  const int nn = static_cast<int>(i % np16);
  if (nn < N) {
    float s = 0.f;
    for (int64_t bb = 0; bb < batch; ++bb) s += wsA[(bb * D16 + cc) * np16 + nn];
    dA[cc * N + nn] = s;
  }
  if (nn == 0 && dD != nullptr) {
    float s = 0.f;
    for (int64_t bb = 0; bb < batch; ++bb) s += wsD[bb * D16 + cc];
    dD[cc] = s;
  }
}

struct Layout {
  size_t ckpt, partB, partC, wsA, wsD, py, ps1, ps2, total;
};
size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }
int64_t slices(int64_t N) { return (N + 15) / 16; }
Layout layout(int64_t batch, int64_t L, int64_t dim, int64_t N) {
  const int64_t ncb = (dim + kCPB - 1) / kCPB, D16 = ncb * kCPB, nt = (L + kTT - 1) / kTT;
  const int64_t nsl = slices(N), NP = 16 * nsl;
  Layout l{};
  size_t off = 0;
  l.ckpt = off;  off += align256(sizeof(float) * static_cast<size_t>(batch * nt * D16 * NP));
  l.partB = off; off += align256(sizeof(float) * static_cast<size_t>(ncb * batch * L * NP));
  l.partC = off; off += align256(sizeof(float) * static_cast<size_t>(ncb * batch * L * NP));
  l.wsA = off;   off += align256(sizeof(float) * static_cast<size_t>(batch * D16 * NP));
  l.wsD = off;   off += align256(sizeof(float) * static_cast<size_t>(batch * D16));
  const size_t part = nsl > 1 ? align256(sizeof(float) * static_cast<size_t>(nsl * batch * L * dim)) : 0;
  l.py = off;    off += part;
  l.ps1 = off;   off += part;
  l.ps2 = off;   off += part;
  l.total = off;
  return l;
}

}  // namespace

size_t scan_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N) {
  return layout(batch, L, dim, N).total;
}

int64_t scan_bwd_grid_blocks(int64_t batch, int64_t dim, int64_t N) {
  return batch * ((dim + kCPB - 1) / kCPB) * slices(N);
}

hipError_t scan_bwd_launch(const ScanBwdArgs& a, hipStream_t stream) {
  const int64_t ncb = (a.dim + kCPB - 1) / kCPB;
  const Layout l = layout(a.batch, a.L, a.dim, a.N);
  const int nsl = static_cast<int>(slices(a.N));
  char* ws = static_cast<char*>(a.workspace);
  BwdParams p{};
  p.x = a.x; p.delta = a.delta; p.B = a.B; p.C = a.C; p.z = a.z; p.dout = a.dout;
  p.A = a.A; p.D = a.D; p.h0 = a.h0; p.dfinal = a.dfinal;
  p.dx = a.dx; p.ddelta = a.ddelta; p.dz = a.dz; p.dh0 = a.dh0;
  p.ckpt = reinterpret_cast<float*>(ws + l.ckpt);
  p.ckpt_in = a.ckpt_in;
  p.partB = reinterpret_cast<float*>(ws + l.partB);
  p.partC = reinterpret_cast<float*>(ws + l.partC);
  p.wsA = reinterpret_cast<float*>(ws + l.wsA);
  p.wsD = reinterpret_cast<float*>(ws + l.wsD);
  if (nsl > 1) {
    p.part_y = reinterpret_cast<float*>(ws + l.py);
    p.part_s1 = reinterpret_cast<float*>(ws + l.ps1);
    p.part_s2 = reinterpret_cast<float*>(ws + l.ps2);
  }
  p.batch = a.batch; p.L = a.L; p.dim = a.dim; p.N = a.N;
  p.ntiles = static_cast<int>((a.L + kTT - 1) / kTT);
  p.ncb = static_cast<int>(ncb);
  p.nsl = nsl;
  p.np16 = 16 * nsl;
  if (a.batch > 0) {
    const dim3 grid(static_cast<unsigned>(ncb * a.batch * nsl));
    if (a.io == 1) {
      if (nsl > 1) hipLaunchKernelGGL((scan_bwd_kernel<uint16_t, true>), grid, dim3(kThreads), 0, stream, p);
      else hipLaunchKernelGGL((scan_bwd_kernel<uint16_t, false>), grid, dim3(kThreads), 0, stream, p);
    } else {
      if (nsl > 1) hipLaunchKernelGGL((scan_bwd_kernel<float, true>), grid, dim3(kThreads), 0, stream, p);
      else hipLaunchKernelGGL((scan_bwd_kernel<float, false>), grid, dim3(kThreads), 0, stream, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nbc = (a.batch * a.L * (p.np16 / 4) + 255) / 256;
    if (nbc > 0) {
      hipLaunchKernelGGL(bwd_reduce_bc, dim3(static_cast<unsigned>(nbc)), dim3(256), 0, stream, p.partB, p.partC,
                         a.dB, a.dC, a.batch, a.L, a.N, p.ncb, p.np16);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    const int64_t nfin = (a.batch * a.L * a.dim + 255) / 256;
    if (nsl > 1 && nfin > 0) {
      if (a.io == 1)
        hipLaunchKernelGGL(bwd_finish<uint16_t>, dim3(static_cast<unsigned>(nfin)), dim3(256), 0, stream, p);
      else
        hipLaunchKernelGGL(bwd_finish<float>, dim3(static_cast<unsigned>(nfin)), dim3(256), 0, stream, p);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  const int64_t nad = (a.dim * p.np16 + 255) / 256;
  hipLaunchKernelGGL(bwd_reduce_ad, dim3(static_cast<unsigned>(nad)), dim3(256), 0, stream, p.wsA, p.wsD, a.dA, a.dD,
                     a.batch, a.dim, a.N, p.ncb, p.np16);
  return hipGetLastError();
}

}  // namespace mssm
