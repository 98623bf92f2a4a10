// kda_internal.h -- host-side launch interface between the C ABI (kda_api.cpp)
// and the kernels (kda_*.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// switches (same values as the KDA_FUSE_* / KDA_GATE_UNBOUNDED constants of the public header)
constexpr uint32_t FUSE_GATE = 1, FUSE_QK_L2NORM = 2, FUSE_BETA_SIGMOID = 4, GATE_UNBOUNDED = 8;

// Where a chunk's tokens are: fixed-length rows (B rows of T tokens) or the varlen
// tables built on the device. A fixed-length launch covers chunks jb .. jb + nc_win - 1
// of every row (all of them unless the workspace holds fewer: see the windowed calls of
// kda_fwd_ex); its slot i is row i / nc_win, chunk jb + i % nc_win of that row.
struct ChunkMap {
  const int2* chunk_tab;   // varlen: [max_chunks] {t0, len}; len = 0 -> unused slot
  const int2* seq_tab;     // varlen: [N] {first chunk, number of chunks}
  const int2* seq_span;    // varlen: [N] {first token, length} (clamped into [0, T])
  const int32_t* seq_order;  // varlen: [N] sequences by chunk count, longest first
  int32_t T;               // tokens per row (fixed) / packed total (varlen)
  int32_t nc_row;          // chunks per row (fixed)
  int32_t jb;              // fixed: first chunk of each row in this launch; varlen: first chunk slot
  int32_t nc_win;          // fixed: chunks of each row in this launch (nc_row unless windowed);
                           // varlen windows: chunk slots per window
  int32_t max_chunks;      // number of chunk slots (of this launch)
  // varlen calls in windows of chunk slots (win >= 0): window win covers slots jb ..
  // jb + nc_win - 1; its sequences are nz_seq[win_first[win]] onwards (kda_sched.hip),
  // nseq is then the launch's sequence capacity nc_win + 1, and a sequence that crosses
  // a window boundary carries its state in fp32 through carry slot (window & 1)
  int32_t win = -1;
  int32_t n_win = 0;
  const int32_t* nz_seq = nullptr;
  const int32_t* win_first = nullptr;
  float* carry = nullptr;  // [2][H][V][K] fp32
  int32_t nseq;            // sequences (B or N)
};

// Segment-parallel state chain. Each row's (fixed length) or sequence's (varlen)
// chunks are cut into nseg segments of ceil(chunks / nseg). Every segment acts on the state as an
// affine map S -> S P + R; the chain kernel computes (P, R) of all segments at once
// (CHAIN_MAPS: R from a zero state, P by running the identity through the recurrence
// without U~), the scan kernel composes them into each segment's initial state, and
// the chain kernel then produces the outputs of all segments at once (CHAIN_OUTPUTS).
enum ChainMode : int32_t { CHAIN_FULL = 0, CHAIN_MAPS = 1, CHAIN_OUTPUTS = 2 };
struct ChainSeg {
  int32_t nseg = 1;        // segments per row or sequence (1: the plain chain)
  int32_t mode = CHAIN_FULL;
  float* maps = nullptr;      // [seqs * nseg][H][256][128] fp32: rows 0-127 R, rows 128-255 P
  float* seg_init = nullptr;  // [seqs * nseg][H][128][128] fp32: each segment's initial state
};

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;
  const uint16_t* beta;
  uint16_t* out;
  const float* A_log;
  const float* dt_bias;
  const void* init_state;
  void* final_state;
  int init_dtype;          // 0 none, 1 bf16, 2 fp32
  int final_dtype;
  float scale;
  float lower_bound;
  int32_t H;
  uint32_t flags;          // KDA_FUSE_* bits (which input processing runs in the kernels), GATE_UNBOUNDED
  ChunkMap map;
  uint8_t* rec;            // chunk records: [max_chunks][H][REC_BYTES]
  ChainSeg seg;
};

hipError_t launch_sched(const int64_t* cu_seqlens, int32_t N, int32_t T, int32_t max_chunks,
                        int2* seq_tab, int2* chunk_tab, int2* seq_span, int32_t* seq_order,
                        hipStream_t stream, int32_t win_chunks = 0, int32_t n_win = 0,
                        int32_t* nz_seq = nullptr, int32_t* win_first = nullptr);
hipError_t launch_intra(const FwdParams& p, hipStream_t stream);
hipError_t launch_chain(const FwdParams& p, hipStream_t stream);
hipError_t launch_scan(const FwdParams& p, int32_t rows, hipStream_t stream);
hipError_t launch_recurrent(const FwdParams& p, const int64_t* cu_seqlens, hipStream_t stream);
// varlen windows: final_state of the sequences without chunks (their initial state, or zeros)
hipError_t launch_empty_states(const FwdParams& p, int32_t N, hipStream_t stream);

}  // namespace kda
