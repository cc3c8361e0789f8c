// entq_internal.h -- layouts shared by the host plan builder and the HIP
// kernels of libentq (never by the CPU oracle).
#pragma once

#include <stdint.h>

#include <vector>

#include "entq.h"

namespace entq {

constexpr uint32_t kProbBits = 12;
constexpr uint32_t kProbScale = 1u << kProbBits;   // M
constexpr uint32_t kLanes = 64;                    // interleaved states per chunk
constexpr uint32_t kStateLow = 1u << 16;           // L
constexpr uint32_t kStateBytes = 4 * kLanes;       // states at the start of a region
constexpr uint32_t kMaxChunkSymbols = 1u << 20;

// Workgroup shape of the decode kernels: kWaves waves, each decoding one
// chunk at a time; all chunks of a workgroup belong to one tensor so they
// share the slot table held in LDS. A workgroup's task is a run of chunks of
// one tensor, decoded in rounds of up to kWaves chunks.
constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;

// Scalar registers a wave of a kWaves-wave kernel may use so that two of its
// workgroups (8 waves per SIMD) are resident on a CU at once. Measured on
// MI355X with workgroups of 16 waves: 80 scalar registers in total (VCC and
// the other reserved ones included) still let two workgroups start
// together, 83 or more let only one start, whatever the LDS size -- and the
// second workgroup then waits until waves of the first exit. The compiler's
// own occupancy estimate does not see this, so the kernels cap the count.
#define ENTQ_TWO_WORKGROUPS_SGPRS __attribute__((amdgpu_num_sgpr(80)))

// The streaming kernel works in blocks of kBlockSteps steps (256 symbols
// per chunk); a tensor can use it when its chunk size is a multiple of the
// block, and, for bf16 output, when a block never crosses a row.
constexpr uint32_t kBlockSteps = 4;
constexpr uint32_t kBlockSyms = kBlockSteps * kLanes;

// Slot table entry, one per slot (4096 per tensor), 8 bytes:
//   lo = f | sym << 24   (f = frequency of the owning symbol, 1..4096, in
//                         bits 0..12; bits 13..23 are zero so that a 24-bit
//                         multiply by lo multiplies by f alone)
//   hi = slot - cum[sym] (the additive term of the decode step)
struct SlotEntry {
    uint32_t lo;
    uint32_t hi;
};

struct DevTensor {
    uint32_t cols;
    uint32_t kind;
    uint32_t pad0, pad1;
};

struct DevChunk {
    uint64_t byte_offset;   // region start in the blob
    uint64_t out_elem;      // absolute output index of the chunk's first symbol
    uint64_t scale_row;     // absolute scale index of the chunk's first symbol
    uint32_t col0;          // column of the chunk's first symbol
    uint32_t n_symbols;
    uint32_t n_words;
    uint32_t status_index;  // position in the caller's chunk index
    uint32_t tensor;
    uint32_t pad;
};
static_assert(sizeof(DevChunk) == 48, "DevChunk layout");

struct DevTask {
    uint32_t first_chunk;   // into the plan's DevChunk array
    uint32_t n_chunks;      // >= 1, consecutive chunks of one tensor
    uint32_t tensor;
    uint32_t pad;
};

// What the host keeps of each tensor of a plan (for launches that need it).
struct HostTensor {
    uint32_t kind, rows, cols, chunk_symbols;
    uint64_t n_symbols;
    int64_t chunk_base;     // its first DevChunk (chunks in element order)
    int64_t n_chunks;
    uint64_t out_elem_offset;
    uint64_t scale_row_offset;
    bool tiles;             // symbols in tile order (ENTQ_LAYOUT_TILES)
};

// In a plan's kinds_mask: some non-empty tensor is in tile order.
constexpr uint32_t kTilesBit = 1u << 31;

}  // namespace entq

// The host-side plan object behind the opaque C handle.
struct entq_plan_s {
    int n_tensors;
    int64_t n_chunks;
    int64_t n_tasks;
    // Tasks are ordered in three groups: [0, n_tasks_rows) have chunk sizes
    // and row lengths that are multiples of kBlockSyms; [n_tasks_rows,
    // n_tasks_blocks) only chunk sizes; the rest neither.
    int64_t n_tasks_rows;
    int64_t n_tasks_blocks;
    // The most chunks any task of [0, n_tasks_rows) / [0, n_tasks_blocks)
    // holds (1: a latency-bound launch, one chunk per workgroup).
    uint32_t max_task_chunks_rows;
    uint32_t max_task_chunks_blocks;
    uint64_t blob_bytes;
    uint64_t out_elems;
    uint64_t scale_rows;
    uint32_t kinds_mask;        // bit k set if some non-empty tensor has kind k; kTilesBit
    const entq::SlotEntry *d_tables;
    const entq::DevTensor *d_tensors;
    const entq::DevChunk *d_chunks;
    const entq::DevTask *d_tasks;
    void *host_staging;         // kept alive until destroy (async copy source)
    std::vector<entq::HostTensor> host_tensors;
    bool adaptive = false;      // chunk regions carry their own tables
    bool mixed_layouts = false; // tile-ordered and row-major tensors together
    void *upload_done = nullptr;  // hipEvent_t recorded after the workspace upload
};

// Launchers implemented in entq_decode.hip.
namespace entq {
enum DecodeMode { kModeCodes = 0, kModeBf16 = 1, kModeSplit = 2 };
int launch_decode(const entq_plan_t *plan, int mode, const void *blob, void *out,
                  const float *scales, const uint8_t *signmant, int32_t *status,
                  void *stream);
// Decode of a plan whose chunks carry their own tables (entq_decode_adaptive.hip).
int launch_decode_adaptive(const entq_plan_t *plan, int mode, const void *blob, void *out,
                           const float *scales, const uint8_t *signmant, int32_t *status,
                           void *stream);
// Fused decode + product with activations (entq_decode_gemm.hip).
// workspace: null, or room for the packed activations (gemm_workspace_bytes).
int launch_decode_gemm(const entq_plan_t *plan, const void *blob, const float *scales,
                       const uint8_t *signmant, const entq_gemm_io *io, int n_rows,
                       uint8_t *workspace, int32_t *status, void *stream);
uint64_t gemm_workspace_bytes(const entq_plan_t *plan, int m);
// Bytes of one tensor's packed activations for m rows (16-row groups,
// 256-byte aligned), and the launch that writes them: tensor t's copy at
// workspace + offsets[t] (fragment of 16-column slice T, group g, lane l at
// element (T * groups + g) * 256 + 4 l; zeros for rows m and beyond).
uint64_t packed_bytes(uint32_t cols, int groups_m);
int launch_pack_activations(const entq_plan_t *plan, const entq_gemm_io *io, int m,
                            const uint64_t *offsets, uint8_t *workspace, void *stream);
// The same product for at most kGemvMaxRows activation rows without matrix
// cores (entq_decode.hip), for plans of at most kGemvMaxTensors tensors whose
// chunks hold whole rows of a multiple of kBlockSyms columns; signmant
// non-null for BF16 exponent streams.
constexpr int kGemvMaxRows = 4;
constexpr int kGemvMaxTensors = 16;
// The decode of a plan whose tensors are all in tile order, into their
// row-major outputs (entq_decode_tiles.hip); mode as for launch_decode.
int launch_tile_decode(const entq_plan_t *plan, int mode, const void *blob, void *out,
                       const float *scales, const uint8_t *signmant, int32_t *status,
                       void *stream);
int launch_decode_gemv(const entq_plan_t *plan, const void *blob, const float *scales,
                       const uint8_t *signmant, const entq_gemm_io *io, int n_rows,
                       int32_t *status, void *stream);
// Workgroups of the decode kernels that fit on the current device at once
// (compute units x workgroups per compute unit); 0 if HIP cannot tell.
int64_t resident_workgroups();
}  // namespace entq
