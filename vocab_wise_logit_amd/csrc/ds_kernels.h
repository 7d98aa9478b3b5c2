// ds_kernels.h -- launch interface between the host library and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ds_device.h"

namespace ds {

// Device workspace of the streaming kernels.  A row is cut into `nparts`
// (vocabulary chunk, part) pieces, each reduced by its own workgroup to a
// partial record; a second kernel merges each row.
struct PartRec {
    float m;      // max of h over the part
    float s;      // sum of exp(h - m) over the part
    int id;       // smallest id attaining m (INT32_MAX when the part is empty)
    int nq;       // ids the part's Gumbel race scored, or -1 when it ran none
    float bz;     // best perturbed score h/tau + G among them
    int be;       // its id (smallest on equal scores)
    float bh;     // its h
    int above;    // keys above the row's threshold window (when the row has one)
};

// The exact threshold's window of one row (threshold output requested): order
// keys [lo, hi] bracketing the row's top_k-th largest key, from a sample of the
// row (lo > hi: no window).  While they stream, the parts count the keys above
// it (PartRec::above) and append the h (raw bits) of the ids inside it to the
// row's key buffer.
struct WinRec {
    uint32_t lo, hi;
    int32_t count;  // keys appended so far (may exceed the buffer: then unusable)
    int32_t pad;
};
constexpr int kWinKeysPerRow = 16384;  // key buffer per row (64 KB)
constexpr int kWinRows = 2048;         // rows per launch the handle's window buffers hold (128 MB)
struct Cand {
    float h;
    int e;
};
constexpr int kRowThreads = 512;
constexpr int kRowThreadsWin = 128;   // the parts kernel with the threshold window
constexpr int kRowU = 4;            // 16-byte pieces per thread per group
constexpr int kWorkParts = 16384;   // parts the workspace holds per launch

struct RowWork {
    PartRec* part;     // [slots * nparts]
    int32_t nparts;    // vocab_chunks * parts_per_chunk
    int32_t ppc;       // parts per chunk
    int64_t cell_base; // first launch-relative cell handled by this launch
    int32_t ncells;    // cells in this launch (<= slots)
    WinRec* win;       // [slots] threshold windows, or nullptr (no window path)
    uint32_t* keys;    // [slots][kWinKeysPerRow] h (raw bits) inside each row's window
};

// Arguments common to one sampler launch (one group of <= 64 requests).
struct SampleArgs {
    const void* c;          // [C, P, V] logits (f32 or bf16)
    const void* u;          // same layout, or nullptr when no request in the call reads it
    int32_t V;
    int32_t rows;           // C
    int32_t top_k;
    int32_t vocab_chunks;   // row kernel only
    uint32_t k0, k1;        // seed halves
    float z0;               // normal quantile used for the first threshold pivot
    int32_t force_fallback; // row kernel: skip the single-pass paths
    int32_t* tokens;        // [C, P]
    float* logprobs;        // [C, P]
    float* thresholds;      // [C, P] or nullptr
    RowWork w;              // streaming kernel workspace (unused by the small kernel)
    // Repetition penalty applied by the streaming parts of the device-parameter
    // kernel before they read their ids (one position per request, so the cell
    // is the row of the logits, of seen and of penalty); nullptr: none.  The
    // logits (c) are then written in place.
    const uint32_t* seen = nullptr;  // [cells, W] seen-id bits
    const float* penalty = nullptr;  // [cells] theta
    int32_t W = 0;                   // ceil(V / 32)
};

// Largest row the wave-per-cell kernel keeps in registers, in dwords per lane.
constexpr int kSmallMaxSlotsBf16 = 16;  // V <= 2046
constexpr int kSmallMaxSlotsF32 = 32;   // V <= 2048
int small_slots_needed(bool bf16, int V);

hipError_t launch_sample_small(bool bf16, const SampleArgs& a, const ReqTable& rq,
                               hipStream_t st);
hipError_t launch_sample_small_dev(bool bf16, const SampleArgs& a, const DevReq& d, hipStream_t st);
hipError_t launch_sample_row(bool bf16, const SampleArgs& a, const ReqTable& rq,
                             hipStream_t st);
hipError_t launch_sample_row_dev(bool bf16, const SampleArgs& a, const DevReq& d, hipStream_t st);

struct GreedyArgs {
    const void* x;      // [n_rows, V]
    int64_t n_rows;
    int32_t V;
    int32_t vocab_chunks;
    int32_t* token;
    float* lse;
    float* logprob;
    float* triples;     // [chunks][n_rows][3] or nullptr
    RowWork w;
};

// Parts per chunk for a launch of `cells` rows (see ds_row.hip).
int row_parts_per_chunk(bool bf16, int V, int chunks, int64_t cells, bool window);

hipError_t launch_greedy_lse(bool bf16, const GreedyArgs& a, hipStream_t st);

// One workgroup per row, no workspace (the draft path when its rows fill the
// GPU).  Needs V and ceil(V / chunks) to be multiples of the ids per 16-byte
// piece, at most kGreedyRowMaxChunks chunks and 16-byte aligned logits.
// 512 threads: the read ceiling of one workgroup per row at the draft path's
// size (256 rows of 496 KB) is highest with 512 threads per workgroup (22.1 us,
// against 23.5 us with 1024), with the same four 16-byte pieces in flight per
// thread.
constexpr int kGreedyRowThreads = 512;
constexpr int kGreedyRowU = 4;  // 16-byte pieces per thread per group
constexpr int kGreedyRowMaxChunks = 64;
bool greedy_rows_fits(bool bf16, int V, int chunks, const void* x);
hipError_t launch_greedy_rows(bool bf16, const GreedyArgs& a, hipStream_t st);

// Repetition penalty of the autoregressive mode, in place: one thread per
// kPenaltyWords seen-mask words.
constexpr int kPenaltyThreads = 256;
constexpr int kPenaltyWords = 2;
constexpr int kPenaltyBatch = 4;  // seen ids whose logits one thread reads at once
struct PenaltyArgs {
    void* logits;           // [n_rows, V], modified in place
    const uint32_t* seen;   // [n_rows, W]
    const float* penalty;   // [n_rows]
    int64_t n_rows;
    int32_t V;
    int32_t W;              // ceil(V / 32)
};
hipError_t launch_repetition_penalty(bool bf16, const PenaltyArgs& a, hipStream_t st);

// Confidence reveal: one workgroup per request, its selected cells sorted in LDS.
constexpr int kRevealThreads = 1024;
constexpr int kRevealCap = 16384;        // cells one request may reveal
constexpr int kMaxRevealPerLaunch = 64;  // requests per launch (kernel-argument table)

struct RevealTable {
    int32_t n;                        // requests in this launch
    int32_t T[kMaxRevealPerLaunch];   // positions of the request
    int32_t k[kMaxRevealPerLaunch];   // cells to reveal
    int64_t off[kMaxRevealPerLaunch]; // first packed position
    int64_t out[kMaxRevealPerLaunch]; // first output slot
};

struct RevealArgs {
    const float* scores;  // [C, P]
    int64_t P;
    int32_t C;
    int32_t* index_out;
    float* score_out;     // or nullptr
};

hipError_t launch_reveal_topk(const RevealArgs& a, const RevealTable& rt, hipStream_t st);

// Measurement aid: n_rows workgroups of `threads` (256, 512 or 1024) threads,
// each reading one row of row_pieces 16-byte pieces once.
hipError_t launch_read_probe(const void* x, int64_t n_rows, int64_t row_pieces, int threads, uint32_t* sink,
                             hipStream_t st);

}  // namespace ds
