// Internal declarations shared by the C-ABI front end and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mssm {

// ---------------------------------------------------------------------------
// Mamba-1 selective scan
// ---------------------------------------------------------------------------
struct ScanArgs {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;       // nullable
  const void* z;        // nullable
  const float* h0;      // nullable
  void* out;
  float* final_state;   // nullable
  void* workspace;
  int64_t batch, L, dim, N;
  int io;               // 0 fp32, 1 bf16
  int K;                // sequence chunks
  int G;                // lanes per channel
  // optional short causal convolution + SiLU in front of the scan; x is then
  // its input (needs G == 16, N == 16 and 16-byte aligned I/O)
  const float* conv_w = nullptr;     // [dim, conv_width]
  const float* conv_b = nullptr;     // [dim], nullable
  const void* conv_init = nullptr;   // [batch, conv_width - 1, dim], nullable
  int conv_width = 0;
  // optional training-mode output: the state entering every 16-step tile,
  // [batch][ceil(L/16)][16 * ceil(dim/16)][16] fp32 (needs G == 16, N == 16)
  float* ckpt = nullptr;
};

// bytes of the checkpoint array the training-mode forward writes and the gradients read
size_t scan_checkpoint_bytes(int64_t batch, int64_t L, int64_t dim);


// Workspace layout for K > 1 (all fp32 / int32, 256-byte aligned blocks):
//   hend [batch][K][dim][N]  state at each chunk's end (chunk 0: true; others: from zero)
//   hin  [batch][K][dim][N]  true state entering each chunk
//   S    [batch][K][dim]     sum of delta over each chunk
//   neg  [batch][K][dim]     chunk contained a negative delta
size_t scan_workspace_bytes(int64_t batch, int64_t dim, int64_t N, int K);

// Enqueue the scan; returns hipSuccess or the launch error.
hipError_t scan_launch(const ScanArgs& a, hipStream_t stream);

// lanes-per-channel values the kernels are built for
bool scan_supported_G(int G, int64_t N);

// Fixed per-device scratch of the entry point that allocates nothing: its size, and its
// address on the device of `stream` (looked up once per device, then kept).
constexpr size_t kScratchBytes = size_t{32} << 20;
hipError_t scratch_address(hipStream_t stream, void** out);

// ---------------------------------------------------------------------------
// Mamba-2 scalar-A multi-head (SSD) form
// ---------------------------------------------------------------------------
struct SSDArgs {
  const void* x;
  const void* delta;
  const void* lam;   // nullable: the Mamba-2 rule; else the Mamba-3 exponential-trapezoidal rule
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* h0;
  void* out;
  float* final_state;
  void* workspace;
  int64_t batch, L, H, P, N, G, Q;
  int64_t R = 1;   // inputs and outputs per channel (MIMO); x, z, out [B, L, H, R, P], B, C [B, L, G, R, N]
};

size_t ssd_workspace_bytes(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int64_t Q);
// headdim and dstate the matrix-core block kernel takes (bf16 I/O), and the MIMO ranks
bool ssd_supported(int64_t P, int64_t N);
bool ssd_rank_supported(int64_t R);
hipError_t ssd_launch(const SSDArgs& a, hipStream_t stream);

// ---------------------------------------------------------------------------
// Token-by-token state update (both forms), state read and written in place
// ---------------------------------------------------------------------------
struct UpdateArgs {
  float* state;
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;       // nullable
  const void* z;        // nullable
  void* out;
  int64_t batch, L, N;
  int64_t dim;          // Mamba-1
  int64_t H, P, G;      // multi-head form
  int io;               // 0 fp32, 1 bf16
  // Mamba-1 only: short causal convolution in front, x being its input
  const float* conv_w = nullptr;   // [dim, conv_width]
  const float* conv_b = nullptr;   // [dim], nullable
  void* conv_state = nullptr;      // [batch, conv_width - 1, dim], read and advanced in place
  const void* conv_in = nullptr;   // with conv_state == nullptr: the window before the first token (nullable)
  void* conv_out = nullptr;        // and the window after the last (nullable: not written)
  int conv_width = 0;
  // multi-head form only: the Mamba-3 exponential-trapezoidal rule
  const void* lam = nullptr;       // [batch, L, H]; nullable = the Mamba-2 rule
  const void* x_prev = nullptr;    // [batch, H, P], the token before the first one; nullable = none
  const void* B_prev = nullptr;    // [batch, G, N], likewise
  const float* omega = nullptr;    // [H, N/2] rotation rates of the state pairs (complex state); nullable
  int64_t rank = 1;                // MIMO inputs and outputs per channel (x, z, out [.., H, rank, P],
                                   // B, C [.., G, rank, N]); > 1 takes no omega
  // with state == nullptr: the state before the first token (nullable: zero) and the one written
  // after the last (nullable: not written), for a whole sequence run through the update kernel
  const float* state_in = nullptr;
  float* state_out = nullptr;
};

hipError_t scan_update_launch(const UpdateArgs& a, hipStream_t stream);
hipError_t ssd_update_launch(const UpdateArgs& a, hipStream_t stream);
// blocks the update kernels launch for `rows` state rows of N states
int64_t update_grid_blocks(int64_t rows, int64_t N);

// ---------------------------------------------------------------------------
// Gradients of the Mamba-1 selective scan (dstate <= 16)
// ---------------------------------------------------------------------------
struct ScanBwdArgs {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;       // nullable
  const void* z;        // nullable
  const float* h0;      // nullable
  const void* dout;
  const float* dfinal;  // nullable
  void* dx;
  void* ddelta;
  float* dA;
  float* dB;
  float* dC;
  float* dD;            // written iff D != nullptr
  void* dz;             // written iff z != nullptr
  float* dh0;           // nullable
  const float* ckpt_in = nullptr;   // nullable: checkpoints from the training-mode forward
  void* workspace;
  int64_t batch, L, dim, N;
  int io;
};

// workspace: per-tile state checkpoints, per-block dB/dC partials, per-row dA/dD partials
size_t scan_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t dim, int64_t N);
// blocks of the main gradient kernel
int64_t scan_bwd_grid_blocks(int64_t batch, int64_t dim, int64_t N);
hipError_t scan_bwd_launch(const ScanBwdArgs& a, hipStream_t stream);

}  // namespace mssm
