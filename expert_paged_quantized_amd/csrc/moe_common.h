// Definitions shared by the HIP kernels and the host runtime of the MoE layer.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace strata {

// Kernel dequant families: int4 affine (group 64 or 128; fp16 compute), MXFP4
// (E2M1 x E8M0; bf16 compute), NVFP4 (E2M1 x E4M3 per 16 x fp32 per matrix;
// fp16 compute).
enum QFormat : int { Q_INT4 = 1, Q_MXFP4 = 2, Q_NVFP4 = 4 };
enum RouterKind : int { R_SOFTMAX = 1, R_SIGMOID = 2 };

// Token tile of the prefill grouped GEMM (rows of one expert segment).
constexpr int kPrefillTM = 128;
// Largest T that takes the decode (split-K GEMV-style) kernels.
constexpr int kDecodeMaxT = 8;
// Rows per tile of a decode forward: one tile per expert up to 4 tokens; above,
// tiles of at most 4 rows (an expert with more takes two), which the
// dot-product decode kernel contracts (its 4-row unit).
constexpr int decode_tile_rows(int T) { return T > 4 ? 4 : (1 << 30); }
// Weight tile: 32 output rows x 64 inputs; one lane owns 16 bytes of codes.
constexpr int kTileRows = 32;
constexpr int kTileK = 64;
constexpr int kTileCodeBytes = 1024;

// One unit of grouped-GEMM work: up to kPrefillTM (prefill) or all (decode)
// rows [row_begin, row_begin + nrows) of the permuted row space, all routed to
// `expert`, whose packed record lives at slot_ptr[slot].  The tiles of one
// expert are consecutive in a list: [group_first, group_first + group_count).
struct Tile {
  int32_t expert;
  int32_t slot;
  int32_t row_begin;
  int32_t nrows;
  int32_t group_first;
  int32_t group_count;
};

// Byte offsets of the regions of one prepacked expert record.
//   w1 = gate and up interleaved per 32-row tile (16 gate rows, then the same
//   16 rows of up), [F/16 tiles][H/64 k-blocks]; w2 = down, [H/32][F/64].
//   codes: 1024 B per tile, lane l holds tile row l%32, inputs 32*(l/32)..+31;
//   scales, per row tile and scale block (a k-block, or a pair of k-blocks for
//   int4 group-128: block index kb >> sshift):
//     int4  128 B (u32 per row: fp16 scale | fp16 bias << 16: the bf16 values
//           times 2^-c of their matrix, exactly; same bytes, re-encoded once),
//     MXFP4  64 B (E8M0 byte per (half, row)),
//     NVFP4 128 B (two E4M3 bytes per (half, row): its two 16-input blocks);
//   gscale (NVFP4 only): fp32 matrix scales of gate, up, down (12 B).
struct RecordLayout {
  int64_t w1_codes, w1_scales, w2_codes, w2_scales, gscale, bytes;
  static int64_t scale_block_bytes(int qf) { return qf == Q_MXFP4 ? 64 : 128; }
  static RecordLayout make(int H, int F, int qf, int sshift) {
    RecordLayout r;
    const int64_t sb = scale_block_bytes(qf);
    const int64_t w1_tiles = int64_t(F / 16) * (H / kTileK);
    const int64_t w2_tiles = int64_t(H / 32) * (F / kTileK);
    r.w1_codes = 0;
    r.w1_scales = r.w1_codes + w1_tiles * kTileCodeBytes;
    r.w2_codes = r.w1_scales + (w1_tiles >> sshift) * sb;
    r.w2_scales = r.w2_codes + w2_tiles * kTileCodeBytes;
    r.gscale = r.w2_scales + (w2_tiles >> sshift) * sb;
    r.bytes = r.gscale + (qf == Q_NVFP4 ? 12 : 0);
    return r;
  }
};

// Arguments of one grouped-GEMM launch (gate+up or down).
struct GemmArgs {
  const void* act;           // gate+up: x [T, H] (MXFP4: bf16 as given; int4, NVFP4:
                             // fp16 x * 2^-xexp[t]); down: h [R, F] (bf16 MXFP4;
                             // int4, NVFP4: fp16 scaled as wexp says)
  const int32_t* gather;     // gate+up: perm (row -> token); down: nullptr (row -> row)
  const Tile* tiles;
  const int32_t* n_tiles_dev;  // device-side tile count, or nullptr to use n_tiles
  int32_t n_tiles;
  const uint8_t* const* slot_ptr;  // device array: slot -> record base
  int64_t off_codes, off_scales;   // region offsets inside a record
  int32_t N;                 // weight output rows (2F for gate+up, H for down)
  int32_t K;                 // reduction length (H or F)
  void* out;                 // gate+up: h [R, F]; down: o fp32 [R, H]
  int32_t out_ld;            // F or H
  int32_t sshift;            // scale block of k-block kb: kb >> sshift
  int64_t off_gscale;        // NVFP4: record offset of this GEMM's fp32 matrix
                             // scales (gate, up: two floats; down: one)
  int32_t ksplit;            // prefill down: K is cut into ksplit equal ranges,
                             // range ks writes its partial sums to out + ks * split_stride
  int64_t split_stride;      // floats between partial-sum planes
  // Power-of-two rescaling of the fp16 formats (int4, NVFP4; unused for
  // MXFP4, whose bf16 operands already have the fp32 exponent range):
  const int32_t* tok_of_row;  // row of the permuted space -> token (perm)
  const int32_t* xexp;        // per token: x reached the GEMM as x * 2^-xexp[t]
  const int32_t* wexp;        // per expert (E + 1 for the shared one) 4 exponents:
                              // kWexpGate, kWexpUp, kWexpDown (fp16 weights hold
                              // w * 2^-c), kWexpH (h row of token t holds
                              // h * 2^-(2 xexp[t] + c))
};
enum WexpIndex : int { kWexpGate = 0, kWexpUp = 1, kWexpDown = 2, kWexpH = 3, kWexpCount = 4 };

// Expert records paged from the pinned host store into device slots by the
// page-in kernel, which reads the store through its device mapping: one
// launch per group of pages instead of one DMA-engine copy per page.
constexpr int kPageJobs = 96;
struct PageBatch {
  const uint8_t* src;        // device address of the pinned host store
  int64_t stride;            // bytes between records, in the store and in the slot pool (multiple of 256)
  uint8_t* const* slot_ptr;  // device array: slot -> record base
  int32_t n;                 // pages in this batch (1 .. kPageJobs)
  int32_t expert[kPageJobs];
  int32_t slot[kPageJobs];
};

// Kernel timing: when the runtime times a single-kernel step it sets this
// per-thread pair, and that kernel is launched with the events attached to the
// dispatch itself (hipExtLaunchKernel), which timestamps the kernel's own
// start and end rather than the queue around it.
struct KernelTimer {
  hipEvent_t start = nullptr, stop = nullptr;
  bool used = false;  // set by the launch that took the events
};
extern thread_local KernelTimer g_ktimer;

// Launches `kernel` on `s`, timed by g_ktimer if set.
template <typename K, typename... Args>
inline void launch_k(K kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t s, Args... args) {
  if (g_ktimer.start && g_ktimer.stop && !g_ktimer.used) {
    g_ktimer.used = true;
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, g_ktimer.start, g_ktimer.stop, 0u, args...);
  } else
    kernel<<<grid, block, shmem, s>>>(args...);
}

}  // namespace strata
