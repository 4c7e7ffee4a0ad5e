// Kernel parameter blocks and host launchers shared between the HIP kernel
// files and the C-ABI layer.  Internal; not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kChunk = 64;   // tokens per chunk
constexpr int kSub = 16;     // tokens per sub-tile

// Per-chunk intermediates written by the intra-chunk kernel and read by the
// state scan: one contiguous record per (b, h, chunk of the current segment),
// record index ((b * H + h) * nc + c).  Element type: fp16 for bf16 inputs,
// fp32 for fp32 inputs (RecOps in kda_common.hpp, which also gives the
// power-of-two factors the fp16 entries carry).  What one record holds
// (D = head dim), as the arrays that the LDS images of the scan and of the
// fused kernel keep (rows padded); in the workspace the same values are stored
// in the unit layout of rec_units below:
//   qg  [64][D]   q^ . Gamma, columns in slot order per 32-group
//   kg  [64][D]   -(k^ . Gamma), columns in slot order (negated, so that the
//                 scan forms V - (K . Gamma) S in one accumulator chain)
//   kdt [D][64]   (k^ . Gamma_last / Gamma)^T, token columns in slot order
//   tb  [64][64]  (I + Diag(beta) StrictTril(A_kk))^{-1} Diag(beta), slot order
//   aq  [64][64]  Tril(A_qk) (diagonal included), slot order
//   gam [D]       Gamma_last, fp32
__host__ __device__ constexpr int round256(int x) { return (x + 255) & ~255; }

// Chunk record in the workspace: 16-byte units in the order the intra-chunk
// kernel's lanes hold them, so that every store instruction of a wave writes
// 1 KB of consecutive bytes, and only what the scan reads.  Offsets in units
// (es = element size: 2 fp16, 4 fp32; a "piece" is 8 elements = es / 2 units):
//   qg, kg  piece (ti, kk, lane) = (ti KS + kk) 64 + lane: row 16 ti + n,
//           channels 32 kk + 8 g4 .. + 7 (n = lane % 16, g4 = lane / 16)
//   kdt     the same pieces, each Kd^T rows 32 kk + n and 32 kk + 16 + n
//           (4 elements each) at token slots 32 (ti / 2) + 8 g4 + 4 (ti % 2)
//   tb      T Diag(beta) rows, slot order: slots 0..31 of rows 0..31, then
//           slots 0..63 of rows 32..63 (the rest is never read)
//   aq      pieces (group, lane) = group 64 + lane, six groups: the column
//           pairs p of row tile ti that reach the diagonal, (ti, p) = (0, 0),
//           (1, 0), (2, 0), (2, 1), (3, 0), (3, 1); a piece holds row
//           16 ti + n at slots 32 p + 8 g4 .. + 7, i.e. blocks 2 p and
//           2 p + 1 side by side.  The scan's K-steps also multiply the upper
//           blocks (0, 1) and (2, 3): the record carries them as zeros.
//   gam     Gamma_last, D fp32
struct RecUnits {
  int qg, kg, kdt, tb, aq, gam, units, bytes;
};
__host__ __device__ constexpr RecUnits rec_units(int es, int D) {
  // qg, kg, kdt: 64 D es / 16 = 4 D es units each; tb: 32 rows x 32 slots +
  // 32 rows x 64 slots = 192 es units; aq: 6 groups x 64 pieces x es / 2;
  // gam: D / 4
  return RecUnits{0,
                  4 * D * es,
                  8 * D * es,
                  12 * D * es,
                  12 * D * es + 192 * es,
                  12 * D * es + 384 * es,
                  12 * D * es + 384 * es + D / 4,
                  round256(16 * (12 * D * es + 384 * es + D / 4))};
}
// aq group of the column pair p of row tile ti (p <= ti / 2), and back
__host__ __device__ constexpr int aq_group(int ti, int p) { return ti < 2 ? ti : 2 * ti - 2 + p; }
__host__ __device__ constexpr int aq_group_tile(int g) { return g < 2 ? g : 2 + (g - 2) / 2; }
__host__ __device__ constexpr int aq_group_pair(int g) { return g < 2 ? 0 : (g - 2) % 2; }

struct ChunkWs {
  char* base;       // record 0
  int64_t rec_bytes;
};

// Pipelined schedule: the records of a launch are counted in segments of
// seg_len chunks (segment s holds chunks [s seg_len, (s + 1) seg_len) of the
// launch, the last one possibly shorter), and producers of every
// kPaceEvery-th chunk wait for the scan's progress (IntraParams::progress).
constexpr int kPaceEvery = 2;
__host__ __device__ constexpr int num_segments(int nc, int seg_len) { return (nc + seg_len - 1) / seg_len; }

// Per-token tensors [B, T, H, d] (token major) or [B, H, T, d] (head first,
// kda_desc.tokens): element offset of token 0 of (b, h), and the distance
// between consecutive tokens of one head (d = 1 for beta).
__host__ __device__ inline int64_t token_base(int head_first, int b, int h, int T, int H, int d) {
  return head_first ? ((int64_t)b * H + h) * T * d : ((int64_t)b * T * H + h) * d;
}
__host__ __device__ inline int64_t token_stride(int head_first, int H, int d) {
  return head_first ? (int64_t)d : (int64_t)H * d;
}

struct IntraParams {
  const void* q;
  const void* k;
  const void* z;
  const void* beta;
  const float* A;
  int B, T, H;
  int head_first;  // q, k, z, beta head first ([B, H, T, ..]) instead of token major
  int t0;          // first token of the segment
  int nc;          // chunks in the segment
  float g_min, q_scale, l2_eps;
  int l2norm;
  int decay;       // 0: K3 bounded map; 1: Kimi Linear softplus map (pairwise diagonal blocks)
  ChunkWs ws;
  // Finished records (count_record), or nullptr: chunk c's record counts in
  // done[s B H + b H + h], s = (t0 / 64 + c) / seg_len its segment of the
  // sequence (seg_len = 0: s = 0); t0 / 64 is then a multiple of seg_len.
  uint32_t* done;
  int seg_len;
  // Chunk order of the workgroups: 0 first chunk first (what a consumer
  // running at the same time needs), 1 last chunk first (a launch whose
  // records are read only after it ends: the records of the first chunks,
  // which the scan reads first, are then the most recently written and the
  // likeliest still to be in the memory-side cache).
  int reverse;
  // Record of chunk c of the launch: ((b H + h) rec_stride + rec_c0 + c).
  // rec_stride = 0 means nc (records of this launch only, rec_c0 = 0).
  int rec_stride, rec_c0;
  // Pacing (pipelined schedule), or progress = nullptr: a workgroup of a
  // chunk c (index in the sequence) with c % kPaceEvery == 0 first waits until
  // the scan of its (b, h) has reached chunk c - lead (progress[b H + h]),
  // so that a record is read a
  // few chunk steps after it is written, while it is still in the memory-side
  // cache.  Performance only: the wait is bounded, and the first one that
  // runs out sets *pacing_off, which ends pacing for the launch.
  const uint32_t* progress;
  uint32_t* pacing_off;
  int lead;
  // clear_words 8-byte words at clear set to zero (grid-strided), or nullptr:
  // the split scan's exchange ring, cleared by the intra-chunk launch that
  // precedes that scan on the same stream
  uint64_t* clear;
  int64_t clear_words;
  uint32_t* clear_status;  // a status word set to zero as well, or nullptr
};

// Status bits a kernel ORs into the workspace's status word (read by
// kda_chunk_fwd_status).
constexpr uint32_t kStatusWaitGaveUp = 1u;  // a bounded wait for records ran out: outputs are invalid
constexpr uint32_t kFlagBadSlot = 1u;       // a state-pool slot was outside [0, n_slots): that sequence skipped

// The scan launch of the pipelined schedule covers every segment; segment
// s's records are complete once done[s B H + b H + h] reaches its number of
// chunks.

struct ScanParams {
  const void* v;        // [B, T, H, D], or nullptr for V = 0 (the transfer of a segment, see kda_chunk_fwd_kcp)
  const void* gate;     // [B, T, H, D] gate logits (input dtype) or nullptr
  const float* rms_w;   // [H, D] or nullptr (weight 1)
  const float* S_in;    // [B, H, D, D] or nullptr (zero state)
  float* S_out;         // [B, H, D, D] (may equal S_in)
  void* o;              // [B, T, H, D] or nullptr
  void* y;              // [B, T, H, D] or nullptr (requires gate)
  int out_f32;          // element type of o and y: 1 fp32, 0 bf16
  float rms_eps;
  int B, T, H;
  int head_first;       // v, gate, o, y head first ([B, H, T, D]) instead of token major
  int t0, nc;           // first token and number of chunks of the segment
  ChunkWs ws;
  const uint32_t* done;  // [B * H]: wait until done[b H + h] >= nc before reading records, or nullptr
  uint32_t* status;     // word OR-ed with kStatusWaitGaveUp when such a wait gives up, or nullptr
  float* snaps;         // [B, n_snap, H, D, D] states at every snap_every-th chunk boundary, or nullptr
  int snap_every;       // chunks between snapshots (snapshot j: state after chunk (j + 1) * snap_every - 1)
  int n_snap;
  // Pipelined schedule (specialised scan kernel only): seg_len > 0, records
  // produced by an intra-chunk launch running beside this one and counted in
  // segments of seg_len chunks of the sequence; done then holds one counter
  // per (segment, b, h), the launch's first at segment t0 / 64 / seg_len.
  // seg_len = 0: all records exist, or done (if not nullptr) is one counter
  // per (b, h).
  int seg_len;
  // [B * H]: the chunk each (b, h) has reached, published every chunk step
  // for the producer's pacing (see IntraParams::progress), or nullptr
  uint32_t* progress;
  // 2: each head's value columns split between two workgroups (see
  // split_supported); xchg then holds their RMSNorm row sums, [B H][2][4][64]
  // 8-byte words zeroed before the launch (needed when y is written)
  int nsplit;
  uint64_t* xchg;
};

// The specialised scan workgroup can split a head's value columns between
// two workgroups for 2-byte inputs at d = 128.
__host__ __device__ constexpr bool split_supported(int in_bytes, int D) { return in_bytes == 2 && D == 128; }
constexpr int kXchgWordsPerHead = 2 * 4 * 64;

// Whether the state after chunk `cg` (global index) is snapshot j, and which.
__device__ __forceinline__ int snapshot_index(const ScanParams& p, int cg) {
  if (p.snaps == nullptr || (cg + 1) % p.snap_every != 0) return -1;
  const int j = (cg + 1) / p.snap_every - 1;
  return j < p.n_snap ? j : -1;
}

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const void* beta;
  const void* z;
  const float* A;
  float* S_pool;          // [n_slots, H, D, D]
  int n_slots;
  const int32_t* slot;    // [n] or nullptr; a slot outside [0, n_slots) is skipped and flagged
  uint32_t* status;       // OR-ed with kFlagBadSlot for such a slot, or nullptr
  const void* gate;       // [n, H, D] or nullptr
  const float* rms_w;     // [H, D] or nullptr
  void* o;                // [n, H, D] or nullptr
  void* y;                // [n, H, D] or nullptr
  int n, H;
  float g_min, q_scale, l2_eps, rms_eps;
  int l2norm;
  int out_f32;
  int decay;              // as IntraParams::decay
};

struct StateIoParams {
  int op;          // 0 zero, 1 import (user -> pool), 2 export (pool -> user)
  int transpose;   // user layout [D_v][D_k] when 1
  int n, H;
  float* pool;            // [n_slots, H, D, D]
  int n_slots;
  const int32_t* slot;    // [n] or nullptr; a slot outside [0, n_slots) is skipped and flagged
  uint32_t* status;       // OR-ed with kFlagBadSlot for such a slot, or nullptr
  float* user;
  int vec16;       // pool and user (if any) 16-byte aligned: copy in 16-byte vectors
};

struct PrepassParams {
  const void* q;
  const void* k;
  const void* z;
  const float* A;
  int B, T, H;
  float g_min, l2_eps;
  int l2norm;
  int decay;   // as IntraParams::decay
  float* G;    // [B, T, H, D] chunk-local inclusive cumulative log-decay
  float* rq;   // [B, T, H]
  float* rk;   // [B, T, H]
};

// Input steps before the core: ShortConv + Swish on q, k, v; Sigmoid on beta.
struct InputPrepParams {
  const void* x[3];        // q, k, v projections [B, T, H * D] (input dtype)
  const float* w[3];       // taps [H * D, W]; tap W - 1 multiplies the current token
  const float* state_in;   // [B, 3, W - 1, H * D] inputs before token 0, oldest first, or nullptr (zeros)
  float* state_out;        // [B, 3, W - 1, H * D] the W - 1 inputs before token T, or nullptr
  void* y[3];              // outputs [B, T, H * D] (input dtype)
  const void* beta_logit;  // [B, T, H] or nullptr
  void* beta;              // [B, T, H]
  int B, T, H, C, W;       // C = H * D (a multiple of 8)
  int tokens_per_block;    // tokens per workgroup row; T when state_out aliases state_in
};

// Host launchers (one per kernel family).  in_f32: inputs are fp32 (else bf16).
hipError_t launch_intra(const IntraParams& p, int D, int in_f32, hipStream_t s);
hipError_t launch_scan(const ScanParams& p, int D, int in_f32, hipStream_t s);
// Fused forward of whole sequences (ip.t0 = p.t0 = 0, p.nc = every chunk; the
// record workspaces are not used).  Only where fused_supported().
bool fused_supported(int D, int in_f32);
hipError_t launch_fused(const IntraParams& ip, const ScanParams& p, int D, int in_f32, hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, int D, int in_f32, hipStream_t s);
hipError_t launch_state_io(const StateIoParams& p, int D, hipStream_t s);
hipError_t launch_prepass(const PrepassParams& p, int D, int in_f32, hipStream_t s);
hipError_t launch_copy_state(const float* src, float* dst, int64_t n_floats, hipStream_t s);
hipError_t launch_input_prep(const InputPrepParams& p, int in_f32, hipStream_t s);
// States of a B x P grid of segments: M, St [B, P, H, D, D] (transfer and
// zero-start state of each segment), S0 [B, H, D, D] or nullptr; writes
// Sin [B, P, H, D, D], the entry state of every segment.
hipError_t launch_kcp_fold(const float* M, const float* St, const float* S0, float* Sin, int B, int P, int H, int D,
                           hipStream_t s);
// dst[i] = identity (D x D) for i < n
hipError_t launch_identity_states(float* dst, int64_t n, int D, hipStream_t s);

}  // namespace kda
