// Host side of the C ABI declared in include/kda.h: argument validation,
// workspace carving, the segment schedules and kernel launches.  No device
// memory is allocated here and no host synchronisation happens (unless
// KDA_DEBUG=1, which synchronises after every launch to localise failures).
// The overlapped schedule keeps, per device, two streams restricted to
// disjoint sets of compute units and a few events, created on first use.
#include "kda.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "kda_params.hpp"

namespace {

using kda::kChunk;

constexpr int32_t kDefaultSegmentTokens = 65536;  // one-stream schedule
constexpr int32_t kDefaultPipeTokens = 8192;      // overlapped schedule
constexpr int32_t kDefaultPipelinedTokens = 128;  // pipelined schedule's record-counting segments

// Test hook (failure handling): KDA_TEST_PRODUCED_SEGMENTS=n makes the
// pipelined schedule launch only the first n of its intra-chunk segments, so
// that the scan's bounded wait for the next one runs out and the status word
// is raised while every kernel still exits normally.  Unset: all segments.
int withheld_segments(int n_seg) {
  const char* e = std::getenv("KDA_TEST_PRODUCED_SEGMENTS");
  if (e == nullptr || e[0] == 0) return n_seg;
  const int n = std::atoi(e);
  return n < 0 ? n_seg : std::min(n, n_seg);
}

// Test hook: KDA_TEST_NO_SPLIT=1 keeps one-stream launches on the unsplit
// scan workgroup, so that tests can compare the two bit for bit.
bool split_disabled() {
  const char* e = std::getenv("KDA_TEST_NO_SPLIT");
  return e != nullptr && e[0] == '1';
}

bool debug_sync() {
  const char* e = std::getenv("KDA_DEBUG");
  return e != nullptr && e[0] == '1';
}

kda_status check_launch(hipError_t e, hipStream_t s) {
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return KDA_ERR_HIP;
  }
  if (debug_sync()) {
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return KDA_ERR_HIP;
    }
  }
  return KDA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_size(kda_dtype t) { return t == KDA_F32 ? 4 : 2; }

// The integer an enum-typed field or argument of the C ABI holds, read as an
// int: a C caller may store any int there, and in C++ reading a value outside
// the enum's range through the enum type is undefined.  Every enum is checked
// this way before it is used as its type.
template <typename E>
int enum_int(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "int-sized enums");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

kda_status validate_desc(const kda_desc* d) {
  if (d == nullptr) return KDA_ERR_NULL_ARG;
  if (d->B < 1 || d->H < 1 || d->T < 0 || d->d_k < 1 || d->d_v < 1 || d->chunk < 1) return KDA_ERR_BAD_SHAPE;
  const int in_dt = enum_int(d->in_dtype), out_dt = enum_int(d->out_dtype);
  if ((in_dt != KDA_F32 && in_dt != KDA_BF16) || (out_dt != KDA_F32 && out_dt != KDA_BF16)) return KDA_ERR_BAD_DTYPE;
  if (d->d_k != d->d_v || (d->d_k != 64 && d->d_k != 128)) return KDA_ERR_UNSUPPORTED;
  if (d->chunk != kChunk) return KDA_ERR_UNSUPPORTED;
  if (!(d->g_min < 0.0f) || d->g_min < -5.5f) return KDA_ERR_UNSUPPORTED;
  if (!(d->l2_eps >= 0.0f) || !(d->rms_eps >= 0.0f)) return KDA_ERR_UNSUPPORTED;
  if (d->segment_tokens < 0 || (d->overlap != 0 && d->overlap != 1) || d->fused < 0 || d->fused > 2)
    return KDA_ERR_BAD_SHAPE;
  const int decay = enum_int(d->decay);
  if (decay != KDA_DECAY_K3 && decay != KDA_DECAY_SOFTPLUS) return KDA_ERR_UNSUPPORTED;
  const int tokens = enum_int(d->tokens);
  if (tokens != KDA_TOKENS_BTHD && tokens != KDA_TOKENS_BHTD) return KDA_ERR_UNSUPPORTED;
  return KDA_OK;
}

// q, k, z, v, gate, o, y and beta head first (kda_desc.tokens)
int head_first(const kda_desc* d) { return enum_int(d->tokens) == KDA_TOKENS_BHTD ? 1 : 0; }

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Whether the byte ranges [a, a + na) and [b, b + nb) share a byte (NULL or
// empty ranges share none).
bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const char* pa = static_cast<const char*>(a);
  const char* pb = static_cast<const char*>(b);
  return pa < pb + nb && pb < pa + na;
}

struct WsLayout {
  size_t off_rec, rec_bytes, off_carry, off_done, off_xchg, total;
};
constexpr int kStatusWords = 64;  // status block ahead of the record counters

// Workspace for a segment of seg_nc chunks: one record per (b, h, chunk), the
// fp32 state carried between segments, one record counter per (segment,
// b, h) of the sequence (the two-stream schedules' hand-over; at most one
// segment per chunk) and the split scan's RMSNorm exchange ring (4 KB per
// head).
WsLayout layout_for(const kda_desc* d, int64_t seg_nc) {
  const int es = (int)elem_size(d->in_dtype);
  const int64_t D = d->d_k;
  const int64_t R = (int64_t)d->B * d->H * seg_nc;
  WsLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  L.rec_bytes = (size_t)kda::rec_units(es, (int)D).bytes;
  L.off_rec = take(R * L.rec_bytes);
  L.off_carry = take((size_t)d->B * d->H * D * D * 4);
  // a 256-byte status block (word 0: kda::kStatus* bits), then the counters
  L.off_done = take(kStatusWords * 4 + (size_t)(((int64_t)d->T + kChunk - 1) / kChunk + 1) * d->B * d->H * 4);
  // the split scan's RMSNorm exchange ring (kda::ScanParams::xchg)
  L.off_xchg = take((size_t)d->B * d->H * kda::kXchgWordsPerHead * 8);
  L.total = o;
  return L;
}

int64_t num_chunks(const kda_desc* d) { return ((int64_t)d->T + kChunk - 1) / kChunk; }

int64_t pipe_chunks(const kda_desc* d) {
  const int64_t toks = d->segment_tokens > 0 ? d->segment_tokens : kDefaultPipeTokens;
  return (toks + kChunk - 1) / kChunk;
}

// The overlapped schedule is worth it when the sequence spans more than one
// segment; its workspace holds two segments of records.
bool pipe_wanted(const kda_desc* d) { return d->overlap != 0 && num_chunks(d) > pipe_chunks(d); }

// The fused kernel (records in LDS, no workspace) serves bf16 inputs with the
// K3 decay, on request only (fused == 2).  One workgroup per (head,
// sequence) carries its head's whole intra-chunk work on one compute unit's
// four producer waves (about 43K cycles per chunk against about 6K for the
// scan's product chain), which measured slower than the two-kernel schedules
// at every B * H tried (96 to 768 pairs), so the library does not pick it by
// itself (fused == 1).
bool fused_wanted(const kda_desc* d) {
  return d->fused == 2 && d->decay == KDA_DECAY_K3 && kda::fused_supported(d->d_k, d->in_dtype == KDA_F32);
}
constexpr size_t kFusedWorkspace = 256;  // what the size query reports for it (nothing is used)

// Pipelined schedule: every record of the sequence stays in the workspace.
// One intra-chunk launch over the whole sequence runs on one library stream,
// producing the records in chunk order, while one scan launch over the
// whole sequence runs on the other and waits inside the kernel for each
// segment's records (short uniform segments, counted per (b, h)).  The scan
// has no per-segment restart (state reload, pipeline fill and drain, launch
// gap), and no record buffer is reused, so correctness never needs a
// producer to wait for the scan (the pacing waits are bounded and for speed
// only).  It needs the specialised scan workgroup (bf16 inputs) and a
// workspace that holds every record; the size query offers that workspace
// up to kPipelinedWorkspaceCap.
constexpr size_t kPipelinedWorkspaceCap = size_t(8) << 30;

// Like the overlapped schedule, only for sequences longer than one segment:
// for shorter ones the intra-chunk kernel on every compute unit followed by
// the scan is faster (B 4, T 4096, H 32: 0.55 ms one stream, 0.71 ms
// pipelined).
bool pipelined_eligible(const kda_desc* d) {
  return d->overlap != 0 && d->in_dtype == KDA_BF16 && !fused_wanted(d) && pipe_wanted(d);
}

// Segment length of the pipelined schedule in chunks (the unit in which the
// scan waits for records): 128 tokens by default.  The producers run at most
// a pacing lead of kPipelinedSlack chunks past the segment ahead of their
// scan, so that a record is read a few chunk steps after it was written,
// while it is still in the memory-side cache, and a short segment lets that
// lead stay short without the scan finding its next segment incomplete.
// Measured on the K3 layer (B 1, T 65,536, H 96; step ms, one box):
// segments of 128 tokens with a lead of 8 chunks 4.29; 192 / 8: 4.31;
// 256 / 8: 4.42-4.60; 512 / 16: 4.70; 64 / 8: 4.57 (an acquire per chunk);
// 128 / 7: 4.81 (the scan waits); 128 / 12: 4.52 (records leave the cache).
int64_t pipelined_chunks(const kda_desc* d) {
  const int64_t toks = d->segment_tokens > 0 ? d->segment_tokens : kDefaultPipelinedTokens;
  return (toks + kChunk - 1) / kChunk;
}
constexpr int kPipelinedSlack = 6;

int pipelined_segments(const kda_desc* d, int64_t seg_nc) {
  return kda::num_segments((int)num_chunks(d), (int)seg_nc);
}

// ---- per-device streams and events of the two-stream schedules --------------
// At most one pair of library streams per device (the intra-chunk stream and
// the scan stream, each restricted to its own compute units) plus five
// events.  The pair is made for the scan's unit count of the call at hand;
// a call with another count first waits for the old pair's work and destroys
// it, so a process that alternates B * H between calls pays that wait (the
// library's own streams only) at each change.  Streams are only created by
// the forward calls, never by the query entry points.
struct StreamPair {
  int n_scan = 0;
  hipStream_t intra = nullptr, scan = nullptr;
};
struct DeviceCtx {
  std::mutex mu;
  bool ready = false;
  int cus = 0;
  hipEvent_t fork = nullptr, join_intra = nullptr, join_scan = nullptr;
  hipEvent_t scan_done[2] = {nullptr, nullptr};
  StreamPair pair;
};
constexpr int kMaxDevices = 64;
DeviceCtx g_dev[kMaxDevices];

// Compute units of the current device (0 if unknown), cached per device.
int device_cus();

// Whether a one-stream call splits each head's scan between two workgroups
// (kda_scan.hip): bf16 inputs at d = 128 and 2 B H workgroups within the
// device's compute units.
bool split_taken(const kda_desc* d) {
  return kda::split_supported((int)elem_size(d->in_dtype), d->d_k) &&
         2 * (int64_t)d->B * d->H <= device_cus() && !split_disabled();
}

// Compute units of the current device (0 if unknown), cached per device.
int device_cus() {
  static std::atomic<int> cached[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 0;
  }
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      (void)hipGetLastError();
      return 0;
    }
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Called with c.mu held.
bool ctx_ready(DeviceCtx& c, int dev) {
  if (c.ready) return true;
  if (hipDeviceGetAttribute(&c.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c.cus < 16) {
    (void)hipGetLastError();
    return false;
  }
  for (hipEvent_t* e : {&c.fork, &c.join_intra, &c.join_scan, &c.scan_done[0],
                        &c.scan_done[1]})
    if (hipEventCreateWithFlags(e, hipEventDisableTiming) != hipSuccess) {
      (void)hipGetLastError();
      return false;
    }
  c.ready = true;
  return true;
}

// Waits for and destroys the device's stream pair.  Called with c.mu held.
bool drop_pair(DeviceCtx& c) {
  bool ok = true;
  for (hipStream_t q : {c.pair.intra, c.pair.scan})
    if (q != nullptr && (hipStreamSynchronize(q) != hipSuccess || hipStreamDestroy(q) != hipSuccess)) ok = false;
  (void)hipGetLastError();
  c.pair = StreamPair{};
  return ok;
}

// The device's stream pair for a scan of n_scan workgroups: the scan stream
// may use the first n_scan compute units of the mask, the intra stream the
// others (consecutive mask bits are spread evenly over the XCDs, measured).
// Called with c.mu held.
bool stream_pair(DeviceCtx& c, int n_scan, hipStream_t* si, hipStream_t* ss) {
  if (c.pair.scan == nullptr || c.pair.n_scan != n_scan) {
    if (c.pair.scan != nullptr && !drop_pair(c)) return false;
    std::vector<uint32_t> ms((c.cus + 31) / 32, 0u), mi((c.cus + 31) / 32, 0u);
    for (int i = 0; i < c.cus; ++i) (i < n_scan ? ms : mi)[i / 32] |= 1u << (i % 32);
    StreamPair p{n_scan, nullptr, nullptr};
    if (hipExtStreamCreateWithCUMask(&p.scan, (uint32_t)ms.size(), ms.data()) != hipSuccess ||
        hipExtStreamCreateWithCUMask(&p.intra, (uint32_t)mi.size(), mi.data()) != hipSuccess) {
      (void)hipGetLastError();
      if (p.scan != nullptr) (void)hipStreamDestroy(p.scan);
      (void)hipGetLastError();
      return false;
    }
    c.pair = p;
  }
  *si = c.pair.intra;
  *ss = c.pair.scan;
  return true;
}

// Which schedule a call with this descriptor and workspace takes on the
// current device: the segment length in chunks, and whether it overlaps.
struct Plan {
  int64_t seg_nc;
  bool overlapped;
  int dev;
  int n_scan;
  bool fused;
  bool pipelined;
  int64_t window;  // pipelined: chunks per window (a multiple of seg_nc, or the whole sequence)
};

// Chunks per window of the pipelined schedule for a workspace of ws_bytes
// bytes: the whole sequence when every record fits, else the largest
// multiple of the segment length whose records fit, or 0 when that is below
// kMinPipelinedWindow chunks (the double-buffered overlapped schedule is then
// at least as fast: with one window of 512 chunks the pipelined windows run
// about as fast as the overlapped schedule's 128-chunk segments).
constexpr int64_t kMinPipelinedWindow = 512;
int64_t pipelined_window(const kda_desc* d, size_t ws_bytes) {
  const int64_t nc = num_chunks(d), seg = pipelined_chunks(d);
  if (ws_bytes >= layout_for(d, nc).total) return nc;
  int64_t lo = 0, hi = nc / seg;  // in segments
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo + 1) / 2;
    if (layout_for(d, mid * seg).total <= ws_bytes)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo * seg >= kMinPipelinedWindow ? lo * seg : 0;
}

// The two library streams can serve B * H scan workgroups on the current
// device (B * H at most 5/8 of its compute units); the streams themselves
// are made at launch time (stream_pair).
bool two_streams(const kda_desc* d, int* dev_out, int* n_scan_out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return false;
  }
  DeviceCtx& c = g_dev[dev];
  std::lock_guard<std::mutex> lock(c.mu);
  const int64_t bh = (int64_t)d->B * d->H;
  if (!(ctx_ready(c, dev) && bh * 8 <= (int64_t)c.cus * 5)) return false;
  *dev_out = dev;
  *n_scan_out = (int)((bh + 7) / 8 * 8);
  return true;
}

// one_stream: the call's stream is being captured into a graph; the
// two-stream schedules then stay out (their scan waits inside the kernel for
// producers that a graph would be free to run after it).
Plan make_plan(const kda_desc* d, size_t ws_bytes, bool one_stream = false) {
  Plan p{};
  p.seg_nc = 1;
  const int64_t nc_total = num_chunks(d);
  if (fused_wanted(d)) {
    p.seg_nc = nc_total < 1 ? 1 : nc_total;
    p.fused = true;
    return p;
  }
  int dev = 0, n_scan = 0;
  const int64_t window = (!one_stream && pipelined_eligible(d)) ? pipelined_window(d, ws_bytes) : 0;
  if (window > 0 && two_streams(d, &dev, &n_scan)) {
    p.pipelined = true;
    p.dev = dev;
    p.n_scan = n_scan;
    p.seg_nc = pipelined_chunks(d);
    p.window = window;
    return p;
  }
  if (!one_stream && pipe_wanted(d) && ws_bytes >= layout_for(d, 2 * pipe_chunks(d)).total &&
      two_streams(d, &dev, &n_scan)) {
    p.seg_nc = pipe_chunks(d);
    p.overlapped = true;
    p.dev = dev;
    p.n_scan = n_scan;
    return p;
  }
  // one stream: the largest segment whose workspace fits
  int64_t lo = 1, hi = nc_total < 1 ? 1 : nc_total;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo + 1) / 2;
    if (layout_for(d, mid).total <= ws_bytes)
      lo = mid;
    else
      hi = mid - 1;
  }
  p.seg_nc = lo;
  return p;
}

// Kinds of the traced kernel launches of a call with this plan, in order
// (KDA_LAUNCH_*); returns how many there are.
int32_t plan_launches(const kda_desc* d, const Plan& p, int32_t* kinds, int32_t max_kinds) {
  int32_t n = 0;
  auto put = [&](int32_t k) {
    if (kinds && n < max_kinds) kinds[n] = k;
    ++n;
  };
  if (p.fused) {
    put(KDA_LAUNCH_FUSED);
  } else if (p.pipelined) {
    for (int64_t c0 = 0; c0 < num_chunks(d); c0 += p.window) {
      put(KDA_LAUNCH_INTRA);
      put(KDA_LAUNCH_SCAN);
    }
  } else {
    const int64_t nc_total = num_chunks(d);
    for (int64_t c0 = 0; c0 < nc_total; c0 += p.seg_nc) {
      put(KDA_LAUNCH_INTRA);
      put(KDA_LAUNCH_SCAN);
    }
  }
  return n;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

kda_status kda_release_resources(void) {
  kda_status st = KDA_OK;
  int prev = -1;
  const bool have_prev = hipGetDevice(&prev) == hipSuccess;
  for (int dev = 0; dev < kMaxDevices; ++dev) {
    DeviceCtx& c = g_dev[dev];
    std::lock_guard<std::mutex> lock(c.mu);
    if (!c.ready && c.pair.scan == nullptr) continue;
    if (hipSetDevice(dev) != hipSuccess) {
      (void)hipGetLastError();
      st = KDA_ERR_HIP;
      continue;
    }
    if (!drop_pair(c)) st = KDA_ERR_HIP;
    for (hipEvent_t* e : {&c.fork, &c.join_intra, &c.join_scan, &c.scan_done[0],
                          &c.scan_done[1]}) {
      if (*e != nullptr && hipEventDestroy(*e) != hipSuccess) st = KDA_ERR_HIP;
      *e = nullptr;
    }
    c.ready = false;
  }
  if (have_prev) (void)hipSetDevice(prev);
  (void)hipGetLastError();
  return st;
}

kda_status kda_chunk_fwd_schedule(const kda_desc* d, size_t ws_bytes, int32_t* segment_tokens,
                                  int32_t* schedule) {
  const kda_status st = validate_desc(d);
  if (st != KDA_OK) return st;
  if (!segment_tokens || !schedule) return KDA_ERR_NULL_ARG;
  if (!fused_wanted(d) && ws_bytes < layout_for(d, 1).total) return KDA_ERR_WORKSPACE;
  const Plan p = make_plan(d, ws_bytes);
  *segment_tokens = (int32_t)(p.seg_nc * kChunk);
  *schedule = p.fused        ? KDA_SCHEDULE_FUSED
              : p.pipelined  ? KDA_SCHEDULE_PIPELINED
              : p.overlapped ? KDA_SCHEDULE_OVERLAPPED
                             : KDA_SCHEDULE_SEGMENTS;
  return KDA_OK;
}

kda_status kda_chunk_fwd_status(const kda_desc* d, const void* ws, size_t ws_bytes, void* stream) {
  const kda_status st = validate_desc(d);
  if (st != KDA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(s) != hipSuccess) {
    (void)hipGetLastError();
    return KDA_ERR_HIP;
  }
  if (ws == nullptr || fused_wanted(d) || ws_bytes < layout_for(d, 1).total || d->T == 0) return KDA_OK;
  const Plan p = make_plan(d, ws_bytes);
  // in the one-stream schedule only the split scan waits (for its other half)
  if (!p.pipelined && !p.overlapped && !split_taken(d)) return KDA_OK;
  const WsLayout L = layout_for(d, p.pipelined ? p.window : p.overlapped ? 2 * pipe_chunks(d) : p.seg_nc);
  uint32_t word = 0;
  if (hipMemcpy(&word, static_cast<const char*>(ws) + L.off_done, sizeof(word), hipMemcpyDeviceToHost) !=
      hipSuccess) {
    (void)hipGetLastError();
    return KDA_ERR_HIP;
  }
  return (word & kda::kStatusWaitGaveUp) ? KDA_ERR_TIMEOUT : KDA_OK;
}

kda_status kda_chunk_fwd_launches(const kda_desc* d, size_t ws_bytes, int32_t* kinds, int32_t max_kinds,
                                  int32_t* n_launches) {
  const kda_status st = validate_desc(d);
  if (st != KDA_OK) return st;
  if (!n_launches || max_kinds < 0 || (max_kinds > 0 && !kinds)) return KDA_ERR_NULL_ARG;
  if (!fused_wanted(d) && ws_bytes < layout_for(d, 1).total) return KDA_ERR_WORKSPACE;
  *n_launches = plan_launches(d, make_plan(d, ws_bytes), kinds, max_kinds);
  return KDA_OK;
}

const char* kda_status_str(kda_status s) {
  switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL_ARG: return "required pointer is NULL";
    case KDA_ERR_BAD_SHAPE: return "invalid size";
    case KDA_ERR_BAD_DTYPE: return "invalid dtype";
    case KDA_ERR_MISALIGNED: return "misaligned pointer";
    case KDA_ERR_UNSUPPORTED: return "unsupported configuration";
    case KDA_ERR_WORKSPACE: return "workspace missing or too small";
    case KDA_ERR_HIP: return "HIP launch failure";
    case KDA_ERR_TIMEOUT: return "an in-kernel wait for chunk records gave up: outputs invalid";
  }
  return "unknown status";
}

kda_status kda_desc_init(kda_desc* d, int32_t B, int32_t T, int32_t H, int32_t head_dim, kda_dtype in_dtype,
                         kda_dtype out_dtype) {
  if (d == nullptr) return KDA_ERR_NULL_ARG;
  std::memset(d, 0, sizeof(*d));
  d->B = B;
  d->T = T;
  d->H = H;
  d->d_k = head_dim;
  d->d_v = head_dim;
  d->chunk = kChunk;
  d->g_min = -5.0f;
  d->q_scale = 1.0f;
  d->l2_eps = 1e-6f;
  d->rms_eps = 1e-6f;
  d->qk_l2norm = 1;
  d->in_dtype = in_dtype;
  d->out_dtype = out_dtype;
  d->segment_tokens = 0;
  d->overlap = 1;
  d->fused = 1;
  d->decay = KDA_DECAY_K3;
  d->tokens = KDA_TOKENS_BTHD;
  return validate_desc(d);
}

size_t kda_chunk_fwd_workspace_size_for(const kda_desc* d, int32_t segment_tokens) {
  if (validate_desc(d) != KDA_OK || segment_tokens < 1) return 0;
  const int64_t seg_nc = ((int64_t)segment_tokens + kChunk - 1) / kChunk;
  return layout_for(d, seg_nc).total;
}

size_t kda_chunk_fwd_workspace_size(const kda_desc* d) {
  if (validate_desc(d) != KDA_OK) return 0;
  if (fused_wanted(d)) return kFusedWorkspace;
  if (pipelined_eligible(d)) {
    // every record when that fits the cap, else the largest window of the
    // pipelined schedule that does
    const size_t all = layout_for(d, num_chunks(d)).total;
    if (all <= kPipelinedWorkspaceCap) return all;
    const int64_t w = pipelined_window(d, kPipelinedWorkspaceCap);
    if (w > 0) return layout_for(d, w).total;
  }
  if (pipe_wanted(d)) return layout_for(d, 2 * pipe_chunks(d)).total;
  const int32_t toks = d->T < kDefaultSegmentTokens ? (d->T > 0 ? d->T : 1) : kDefaultSegmentTokens;
  return kda_chunk_fwd_workspace_size_for(d, toks);
}

}  // extern "C"

namespace {

// Records events[2i] / events[2i+1] around the i-th launch while they last.
struct Tracer {
  void* const* ev;
  int32_t n;
  int32_t i = 0;
  void before(hipStream_t s) {
    if (ev && 2 * i + 1 < n) (void)hipEventRecord(static_cast<hipEvent_t>(ev[2 * i]), s);
  }
  void after(hipStream_t s) {
    if (ev && 2 * i + 1 < n) (void)hipEventRecord(static_cast<hipEvent_t>(ev[2 * i + 1]), s);
    ++i;
  }
};

struct Snapshots {
  float* ptr;  // [B, n, H, d_k, d_v] or nullptr
  int every;   // chunks between snapshots
  int n;
};

kda_status chunk_fwd_impl(const kda_desc* d, const void* q, const void* k, const void* v, const void* beta,
                          const void* z, const float* A, const float* S0, const void* gate, const float* rms_w,
                          void* o, void* y, float* S_T, void* ws, size_t ws_bytes, void* stream, Tracer tr,
                          Snapshots snap = Snapshots{nullptr, 1, 0}, bool v_optional = false) {
  kda_status st = validate_desc(d);
  if (st != KDA_OK) return st;
  if (!o && !y && !S_T && !snap.ptr) return KDA_ERR_NULL_ARG;
  if (d->T == 0) {  // nothing to read: S_T = S0 (or zero); inputs may be NULL
    if ((S0 && !aligned(S0, 4)) || (S_T && !aligned(S_T, 4))) return KDA_ERR_MISALIGNED;
    if (S_T && S_T != S0)
      return check_launch(kda::launch_copy_state(S0, S_T, (int64_t)d->B * d->H * d->d_k * d->d_v,
                                                 static_cast<hipStream_t>(stream)),
                          static_cast<hipStream_t>(stream));
    return KDA_OK;
  }
  if (!q || !k || (!v && !v_optional) || !beta || !z || !A) return KDA_ERR_NULL_ARG;  // no V: V = 0
  if (y && !gate) return KDA_ERR_NULL_ARG;
  const size_t es = elem_size(d->in_dtype);
  for (const void* p : {q, k, v, z, (const void*)o, (const void*)y, gate, (const void*)ws})
    if (p && !aligned(p, 16)) return KDA_ERR_MISALIGNED;
  if (!aligned(beta, es) || !aligned(A, 4) || (S0 && !aligned(S0, 4)) || (S_T && !aligned(S_T, 4)) ||
      (rms_w && !aligned(rms_w, 4)))
    return KDA_ERR_MISALIGNED;
  {
    // o, y and S_T overlap no input and no other output (S_T may equal S0)
    const size_t es_out = elem_size(d->out_dtype);
    const size_t row = (size_t)d->B * d->T * d->H;
    const size_t sb = (size_t)d->B * d->H * d->d_k * d->d_v * 4;
    const void* ins[9] = {q, k, v, beta, z, A, S0, gate, rms_w};
    const size_t in_b[9] = {row * d->d_k * es, row * d->d_k * es, row * d->d_v * es, row * es, row * d->d_k * es,
                            (size_t)d->H * 4, sb, row * d->d_v * es, (size_t)d->H * d->d_v * 4};
    const void* outs[3] = {o, y, S_T};
    const size_t out_b[3] = {row * d->d_v * es_out, row * d->d_v * es_out, sb};
    for (int i = 0; i < 3; ++i) {
      for (int j = 0; j < 9; ++j)
        if (!(i == 2 && j == 6 && outs[i] == ins[j]) && ranges_overlap(outs[i], out_b[i], ins[j], in_b[j]))
          return KDA_ERR_UNSUPPORTED;
      for (int j = i + 1; j < 3; ++j)
        if (ranges_overlap(outs[i], out_b[i], outs[j], out_b[j])) return KDA_ERR_UNSUPPORTED;
    }
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int D = d->d_k;
  const int in_f32 = d->in_dtype == KDA_F32;
  const int out_f32 = d->out_dtype == KDA_F32;
  const int64_t nc_total = num_chunks(d);
  const bool fused = fused_wanted(d);
  if (!fused && (!ws || ws_bytes < layout_for(d, 1).total)) return KDA_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);

  // one segment: records of chunks [c0, c0 + nc) in `recs`; state S_in -> S_out
  // seg_len: the pipelined schedule's counting segments (the record counters
  // of one launch over several segments), 0 for one counter per (b, h)
  auto launch_intra = [&](int64_t c0, int nc, const kda::ChunkWs& recs, hipStream_t st_, uint32_t* done = nullptr,
                          int rec_stride = 0, int rec_c0 = 0, int seg_len = 0,
                          const uint32_t* progress = nullptr, uint32_t* pacing_off = nullptr, int lead = 0,
                          uint64_t* clear = nullptr, int64_t clear_words = 0, uint32_t* clear_status = nullptr) {
    kda::IntraParams ip{};
    ip.head_first = head_first(d);
    ip.q = q;
    ip.k = k;
    ip.z = z;
    ip.beta = beta;
    ip.A = A;
    ip.B = d->B;
    ip.T = d->T;
    ip.H = d->H;
    ip.t0 = (int)(c0 * kChunk);
    ip.nc = nc;
    ip.g_min = d->g_min;
    ip.q_scale = d->q_scale;
    ip.l2_eps = d->l2_eps;
    ip.l2norm = d->qk_l2norm;
    ip.decay = d->decay;
    ip.ws = recs;
    ip.done = done;
    ip.seg_len = seg_len;
    // nothing reads these records before the launch ends (one stream):
    // last chunk first (measured on the prefill workload: scan 0.231 ->
    // 0.221 ms, whole call 0.453 -> 0.444 ms median)
    ip.reverse = done == nullptr ? 1 : 0;
    ip.rec_stride = rec_stride;
    ip.rec_c0 = rec_c0;
    ip.progress = progress;
    ip.pacing_off = pacing_off;
    ip.lead = lead;
    ip.clear = clear;
    ip.clear_words = clear_words;
    ip.clear_status = clear_status;
    tr.before(st_);
    const kda_status r = check_launch(kda::launch_intra(ip, D, in_f32, st_), st_);
    tr.after(st_);
    return r;
  };
  auto launch_scan = [&](int64_t c0, int nc, const kda::ChunkWs& recs, const float* S_in, float* S_out,
                         hipStream_t st_, const uint32_t* done = nullptr, int seg_len = 0,
                         uint32_t* status = nullptr, uint32_t* progress = nullptr, uint64_t* xchg = nullptr) {
    kda::ScanParams sp{};
    sp.head_first = head_first(d);
    sp.v = v;
    sp.gate = y ? gate : nullptr;
    sp.rms_w = rms_w;
    sp.S_in = S_in;
    sp.S_out = S_out;
    sp.o = o;  // NULL when only S_T (or only y) is requested
    sp.y = y;
    sp.out_f32 = out_f32;
    sp.rms_eps = d->rms_eps;
    sp.B = d->B;
    sp.T = d->T;
    sp.H = d->H;
    sp.t0 = (int)(c0 * kChunk);
    sp.nc = nc;
    sp.ws = recs;
    sp.done = done;
    sp.status = status;
    sp.snaps = snap.n > 0 ? snap.ptr : nullptr;
    sp.snap_every = snap.every;
    sp.n_snap = snap.n;
    sp.seg_len = seg_len;
    sp.progress = progress;
    sp.nsplit = xchg != nullptr ? 2 : 1;
    sp.xchg = xchg;
    tr.before(st_);
    const kda_status r = check_launch(kda::launch_scan(sp, D, in_f32, st_), st_);
    tr.after(st_);
    return r;
  };

  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &capture) != hipSuccess) {
    (void)hipGetLastError();
    capture = hipStreamCaptureStatusNone;
  }
  const Plan plan = make_plan(d, ws_bytes, capture != hipStreamCaptureStatusNone);

  // ---- fused schedule: one launch, records in LDS
  if (plan.fused) {
    kda::IntraParams ip{};
    ip.head_first = head_first(d);
    ip.q = q;
    ip.k = k;
    ip.z = z;
    ip.beta = beta;
    ip.A = A;
    ip.B = d->B;
    ip.T = d->T;
    ip.H = d->H;
    ip.t0 = 0;
    ip.nc = (int)nc_total;
    ip.g_min = d->g_min;
    ip.q_scale = d->q_scale;
    ip.l2_eps = d->l2_eps;
    ip.l2norm = d->qk_l2norm;
    ip.decay = d->decay;
    kda::ScanParams sp{};
    sp.head_first = head_first(d);
    sp.v = v;
    sp.gate = y ? gate : nullptr;
    sp.rms_w = rms_w;
    sp.S_in = S0;
    sp.S_out = S_T;  // NULL: the final state is not stored
    sp.o = o;
    sp.y = y;
    sp.out_f32 = out_f32;
    sp.rms_eps = d->rms_eps;
    sp.B = d->B;
    sp.T = d->T;
    sp.H = d->H;
    sp.t0 = 0;
    sp.nc = (int)nc_total;
    sp.snaps = snap.n > 0 ? snap.ptr : nullptr;
    sp.snap_every = snap.every;
    sp.n_snap = snap.n;
    tr.before(s);
    const kda_status r = check_launch(kda::launch_fused(ip, sp, D, in_f32, s), s);
    tr.after(s);
    return r;
  }

  // ---- pipelined schedule (see pipelined_eligible): every record in the
  // workspace, [B H][nc_total]; one intra-chunk launch over the sequence on
  // one library stream (records in chunk order, each counted in its
  // segment's counter), one scan launch over the sequence on the other,
  // which waits inside the kernel for each segment's record counters (zeroed
  // on the caller's stream first).
  if (plan.pipelined) {
    const int64_t window = plan.window;
    const WsLayout L = layout_for(d, window);
    DeviceCtx& c = g_dev[plan.dev];
    std::lock_guard<std::mutex> lock(c.mu);
    hipStream_t si = nullptr, ss = nullptr;
    if (!stream_pair(c, plan.n_scan, &si, &ss)) return KDA_ERR_HIP;
    kda::ChunkWs recs{};
    recs.base = base + L.off_rec;
    recs.rec_bytes = (int64_t)L.rec_bytes;
    uint32_t* status = reinterpret_cast<uint32_t*>(base + L.off_done);
    uint32_t* done = status + kStatusWords;
    auto ok = [](hipError_t e) {
      if (e == hipSuccess) return true;
      (void)hipGetLastError();
      return false;
    };
    const int64_t bh_n = (int64_t)d->B * d->H;
    const int seg_len = (int)plan.seg_nc;
    const int n_seg = pipelined_segments(d, plan.seg_nc);
    // status words (word 1: pacing off), the segment counters, then the
    // scan's progress per (b, h), all zeroed on the caller's stream first
    uint32_t* progress = done + n_seg * bh_n;
    st = check_launch(kda::launch_copy_state(nullptr, reinterpret_cast<float*>(status),
                                             kStatusWords + (n_seg + 1) * bh_n, s),
                      s);
    if (st != KDA_OK) return st;
    if (!ok(hipEventRecord(c.fork, s)) || !ok(hipStreamWaitEvent(si, c.fork, 0)) ||
        !ok(hipStreamWaitEvent(ss, c.fork, 0)))
      return KDA_ERR_HIP;
    float* S_run = S_T ? S_T : reinterpret_cast<float*>(base + L.off_carry);
    const float* S_in = S0;
    // pacing lead: a segment and kPipelinedSlack chunks (a producer waiting
    // for the scan never holds back a record the scan is waiting for)
    const int lead = seg_len + kPipelinedSlack;
    // Windows of `window` chunks (one window when every record fits): per
    // window one intra-chunk launch and one scan launch, the state carried
    // from window to window.  The records of a window reuse the workspace,
    // so a window's intra-chunk launch first waits, through an event, for
    // the previous window's scan.  Each intra-chunk launch is enqueued
    // before its scan: should the two library streams share a hardware queue
    // (their work then runs in enqueue order), every scan still finds its
    // records written instead of waiting for producers queued behind it.
    const int64_t produced = (int64_t)withheld_segments(n_seg) * seg_len;  // chunks the producers cover
    int w = 0;
    for (int64_t c0 = 0; c0 < nc_total; c0 += window, ++w) {
      const int nw = (int)std::min<int64_t>(window, nc_total - c0);
      if (w > 0 && !ok(hipStreamWaitEvent(si, c.scan_done[(w - 1) & 1], 0))) return KDA_ERR_HIP;
      const int nc_prod = (int)std::max<int64_t>(0, std::min<int64_t>(nw, produced - c0));
      if (nc_prod > 0) {
        st = launch_intra(c0, nc_prod, recs, si, done, nw, 0, seg_len, progress, status + 1, lead);
        if (st != KDA_OK) return st;
      }
      st = launch_scan(c0, nw, recs, S_in, S_run, ss, done, seg_len, status, progress);
      if (st != KDA_OK) return st;
      S_in = S_run;
      if (c0 + window < nc_total && !ok(hipEventRecord(c.scan_done[w & 1], ss))) return KDA_ERR_HIP;
    }
    if (!ok(hipEventRecord(c.join_intra, si)) || !ok(hipEventRecord(c.join_scan, ss)) ||
        !ok(hipStreamWaitEvent(s, c.join_intra, 0)) || !ok(hipStreamWaitEvent(s, c.join_scan, 0)))
      return KDA_ERR_HIP;
    return KDA_OK;
  }

  // ---- overlapped schedule: intra(s + 1) on one stream while scan(s) runs on
  // another.  The scan of segment s does not wait for the intra launch of
  // segment s through an event (a cross-stream dependency costs ≈50 µs per
  // segment here); it waits inside the kernel for the segment's record
  // counter (count_record / wait_records), which the intra workgroups raise
  // as their device-scope record stores complete.  Reusing a record buffer
  // (segment s + 2) still waits for the scan that read it through an event.
  // The counters are zeroed on the caller's stream first.
  if (plan.overlapped) {
    const int64_t seg_nc = plan.seg_nc;
    const WsLayout L = layout_for(d, 2 * seg_nc);
    DeviceCtx& c = g_dev[plan.dev];
    std::lock_guard<std::mutex> lock(c.mu);
    hipStream_t si = nullptr, ss = nullptr;
    if (stream_pair(c, plan.n_scan, &si, &ss)) {
      const size_t buf_bytes = (size_t)d->B * d->H * seg_nc * L.rec_bytes;
      kda::ChunkWs bufs[2];
      for (int j = 0; j < 2; ++j) {
        bufs[j].base = base + L.off_rec + j * buf_bytes;
        bufs[j].rec_bytes = (int64_t)L.rec_bytes;
      }
      float* carry = reinterpret_cast<float*>(base + L.off_carry);
      float* S_run = S_T ? S_T : carry;
      uint32_t* status = reinterpret_cast<uint32_t*>(base + L.off_done);
      uint32_t* done = status + kStatusWords;
      auto ok = [](hipError_t e) {
        if (e == hipSuccess) return true;
        (void)hipGetLastError();
        return false;
      };
      const int64_t n_seg = (nc_total + seg_nc - 1) / seg_nc;
      // zero bits: the fp32 fill of a state copy from nothing
      const int64_t bh_n = (int64_t)d->B * d->H;
      st = check_launch(
          kda::launch_copy_state(nullptr, reinterpret_cast<float*>(status), kStatusWords + n_seg * bh_n, s), s);
      if (st != KDA_OK) return st;
      if (!ok(hipEventRecord(c.fork, s)) || !ok(hipStreamWaitEvent(si, c.fork, 0)) ||
          !ok(hipStreamWaitEvent(ss, c.fork, 0)))
        return KDA_ERR_HIP;
      const float* S_in = S0;
      int64_t seg = 0;
      for (int64_t c0 = 0; c0 < nc_total; c0 += seg_nc, ++seg) {
        const int nc = (int)((nc_total - c0) < seg_nc ? (nc_total - c0) : seg_nc);
        const int j = (int)(seg & 1);
        // buffer j was last read by the scan two segments back
        if (seg >= 2 && !ok(hipStreamWaitEvent(si, c.scan_done[j], 0))) return KDA_ERR_HIP;
        st = launch_intra(c0, nc, bufs[j], si, done + seg * bh_n);
        if (st != KDA_OK) return st;
        st = launch_scan(c0, nc, bufs[j], S_in, S_run, ss, done + seg * bh_n, 0, status);
        if (st != KDA_OK) return st;
        if (!ok(hipEventRecord(c.scan_done[j], ss))) return KDA_ERR_HIP;
        S_in = S_run;
      }
      if (!ok(hipEventRecord(c.join_intra, si)) || !ok(hipEventRecord(c.join_scan, ss)) ||
          !ok(hipStreamWaitEvent(s, c.join_intra, 0)) || !ok(hipStreamWaitEvent(s, c.join_scan, 0)))
        return KDA_ERR_HIP;
      return KDA_OK;
    }
    return KDA_ERR_HIP;  // unreachable: make_plan created the pair
  }

  // ---- one stream: segments in turn.  With the device's compute units to
  // spare (2 B H of them), each head's scan is split between two workgroups
  // by value columns (kda_scan.hip); the first intra-chunk launch clears the
  // split's exchange ring.
  const int64_t seg_nc = plan.seg_nc;
  const WsLayout L = layout_for(d, seg_nc);
  kda::ChunkWs cw{};
  cw.base = base + L.off_rec;
  cw.rec_bytes = (int64_t)L.rec_bytes;
  float* carry = reinterpret_cast<float*>(base + L.off_carry);
  float* S_run = S_T ? S_T : carry;
  const float* S_in = S0;
  const int64_t bh_n = (int64_t)d->B * d->H;
  // the split's bounded wait for the other half reports through the status
  // word, cleared by the first intra-chunk launch with the exchange ring
  uint64_t* xchg = nullptr;
  uint32_t* status = nullptr;
  if (split_taken(d)) {
    xchg = reinterpret_cast<uint64_t*>(base + L.off_xchg);
    status = reinterpret_cast<uint32_t*>(base + L.off_done);
  }
  for (int64_t c0 = 0; c0 < nc_total; c0 += seg_nc) {
    const int nc = (int)((nc_total - c0) < seg_nc ? (nc_total - c0) : seg_nc);
    const bool first = xchg != nullptr && c0 == 0;
    const bool clear = first && y != nullptr;
    st = launch_intra(c0, nc, cw, s, nullptr, 0, 0, 0, nullptr, nullptr, 0, clear ? xchg : nullptr,
                      clear ? bh_n * kda::kXchgWordsPerHead : 0, first ? status : nullptr);
    if (st != KDA_OK) return st;
    st = launch_scan(c0, nc, cw, S_in, S_run, s, nullptr, 0, status, nullptr, xchg);
    if (st != KDA_OK) return st;
    S_in = S_run;
  }
  return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_chunk_fwd(const kda_desc* d, const void* q, const void* k, const void* v, const void* beta,
                         const void* z, const float* A, const float* S0, const void* gate, const float* rms_w,
                         void* o, void* y, float* S_T, void* ws, size_t ws_bytes, void* stream) {
  return chunk_fwd_impl(d, q, k, v, beta, z, A, S0, gate, rms_w, o, y, S_T, ws, ws_bytes, stream,
                        Tracer{nullptr, 0});
}

}  // extern "C"

// ---- entry point for callers that cannot allocate ---------------------------
// kda_chunk_fwd_noalloc keeps its chunk records and carried state in this
// file-scope device array instead of a caller workspace.  In host code the
// name is only a host-side stand-in: the array's device address, which differs
// per GPU, is taken once per device with hipGetSymbolAddress and only that
// address is handed to kernels.
static constexpr size_t kNoAllocScratchBytes = KDA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (taken on the first call
// on each device, with that device current).
kda_status scratch_on_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return KDA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return KDA_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KDA_OK;
}
}  // namespace

extern "C" {

kda_status kda_chunk_fwd_noalloc(const kda_desc* d, const void* q, const void* k, const void* v, const void* beta,
                                 const void* z, const float* A, const float* S0, const void* gate,
                                 const float* rms_w, void* o, void* y, float* S_T, void* stream) {
  const kda_status st = validate_desc(d);
  if (st != KDA_OK) return st;
  // the one-stream schedule: no library streams or events, segments in turn
  kda_desc one = *d;
  one.overlap = 0;
  one.fused = 0;
  if (d->T > 0 && layout_for(&one, 1).total > kNoAllocScratchBytes) return KDA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (d->T > 0) {
    const kda_status sst = scratch_on_current_device(&ws);
    if (sst != KDA_OK) return sst;
  }
  return chunk_fwd_impl(&one, q, k, v, beta, z, A, S0, gate, rms_w, o, y, S_T, ws, d->T > 0 ? kNoAllocScratchBytes : 0,
                        stream, Tracer{nullptr, 0});
}

kda_status kda_chunk_fwd_traced(const kda_desc* d, const void* q, const void* k, const void* v, const void* beta,
                                const void* z, const float* A, const float* S0, const void* gate,
                                const float* rms_w, void* o, void* y, float* S_T, void* ws, size_t ws_bytes,
                                void* stream, void* const* events, int32_t n_events) {
  return chunk_fwd_impl(d, q, k, v, beta, z, A, S0, gate, rms_w, o, y, S_T, ws, ws_bytes, stream,
                        Tracer{events, n_events < 0 ? 0 : n_events});
}

kda_status kda_chunk_fwd_snapshots(const kda_desc* d, const void* q, const void* k, const void* v,
                                   const void* beta, const void* z, const float* A, const float* S0,
                                   const void* gate, const float* rms_w, void* o, void* y, float* S_T,
                                   float* snapshots, int32_t every_chunks, void* ws, size_t ws_bytes, void* stream) {
  const kda_status st = validate_desc(d);
  if (st != KDA_OK) return st;
  if (every_chunks < 1) return KDA_ERR_BAD_SHAPE;
  const int32_t n = d->T / (kChunk * every_chunks);
  if (n == 0) {  // no boundary to snapshot: the plain forward, if any output is asked for
    if (!o && !y && !S_T) return KDA_OK;
    return chunk_fwd_impl(d, q, k, v, beta, z, A, S0, gate, rms_w, o, y, S_T, ws, ws_bytes, stream,
                          Tracer{nullptr, 0});
  }
  if (!snapshots) return KDA_ERR_NULL_ARG;
  if (!aligned(snapshots, 4)) return KDA_ERR_MISALIGNED;
  return chunk_fwd_impl(d, q, k, v, beta, z, A, S0, gate, rms_w, o, y, S_T, ws, ws_bytes, stream, Tracer{nullptr, 0},
                        Snapshots{snapshots, every_chunks, n});
}

kda_status kda_input_prep(const kda_desc* d, int32_t conv_width, const void* xq, const void* xk, const void* xv,
                          const void* beta_logits, const float* wq, const float* wk, const float* wv,
                          const float* state_in, float* state_out, void* q, void* k, void* v, void* beta,
                          void* stream) {
  const kda_status st = validate_desc(d);
  if (st != KDA_OK) return st;
  if (conv_width < 1 || conv_width > 4 || head_first(d)) return KDA_ERR_UNSUPPORTED;
  if ((beta_logits == nullptr) != (beta == nullptr)) return KDA_ERR_NULL_ARG;
  const size_t es = elem_size(d->in_dtype);
  for (const float* p : {state_in, (const float*)state_out})
    if (p && !aligned(p, 4)) return KDA_ERR_MISALIGNED;
  kda::InputPrepParams p{};
  p.B = d->B;
  p.T = d->T;
  p.H = d->H;
  p.C = d->H * d->d_k;
  p.W = conv_width;
  p.state_in = conv_width > 1 ? state_in : nullptr;
  p.state_out = conv_width > 1 ? state_out : nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d->T == 0) return check_launch(kda::launch_input_prep(p, d->in_dtype == KDA_F32, s), s);
  if (!xq || !xk || !xv || !wq || !wk || !wv || !q || !k || !v) return KDA_ERR_NULL_ARG;
  for (const void* ptr : {xq, xk, xv, (const void*)q, (const void*)k, (const void*)v})
    if (!aligned(ptr, 16)) return KDA_ERR_MISALIGNED;
  if (!aligned(wq, 4) || !aligned(wk, 4) || !aligned(wv, 4) || (beta && (!aligned(beta, es) || !aligned(beta_logits, es))))
    return KDA_ERR_MISALIGNED;
  // No output may overlap an input it does not equal: a token block re-reads
  // the conv_width - 1 inputs before it, which a neighbouring block's outputs
  // would already have replaced.  beta may equal beta_logits (elementwise);
  // state_out may equal state_in (handled by a single token block).
  {
    const size_t xb = (size_t)d->B * d->T * d->H * d->d_k * es;
    const size_t sb = (size_t)d->B * 3 * (conv_width - 1) * d->H * d->d_k * 4;
    const size_t bb = (size_t)d->B * d->T * d->H * es;
    const void* ins[5] = {xq, xk, xv, conv_width > 1 ? state_in : nullptr, beta_logits};
    const size_t in_b[5] = {xb, xb, xb, sb, bb};
    const void* outs[5] = {q, k, v, conv_width > 1 ? state_out : nullptr, beta};
    const size_t out_b[5] = {xb, xb, xb, sb, bb};
    for (int i = 0; i < 5; ++i)
      for (int j = 0; j < 5; ++j) {
        const bool same_ok = outs[i] == ins[j] && ((i == 3 && j == 3) || (i == 4 && j == 4));
        if (!same_ok && ranges_overlap(outs[i], out_b[i], ins[j], in_b[j])) return KDA_ERR_UNSUPPORTED;
      }
    for (int i = 0; i < 5; ++i)
      for (int j = i + 1; j < 5; ++j)
        if (ranges_overlap(outs[i], out_b[i], outs[j], out_b[j])) return KDA_ERR_UNSUPPORTED;
  }
  p.x[0] = xq;
  p.x[1] = xk;
  p.x[2] = xv;
  p.w[0] = wq;
  p.w[1] = wk;
  p.w[2] = wv;
  p.y[0] = q;
  p.y[1] = k;
  p.y[2] = v;
  p.beta_logit = beta_logits;
  p.beta = beta;
  // in place: one block of tokens per channel group, so that the state is
  // read before it is overwritten by the same thread
  p.tokens_per_block = (p.state_out != nullptr && p.state_out == p.state_in) ? d->T : 128;
  return check_launch(kda::launch_input_prep(p, d->in_dtype == KDA_F32, s), s);
}

namespace {
// KCP: n_parts equal segments per sequence, each a multiple of the chunk.
bool kcp_shape(const kda_desc* d, int32_t n_parts, kda_desc* inner) {
  if (n_parts < 2 || d->T % (n_parts * kChunk) != 0 || (int64_t)d->B * n_parts > 0x7fffffff) return false;
  *inner = *d;
  inner->B = d->B * n_parts;
  inner->T = d->T / n_parts;
  return true;
}
size_t kcp_state_bytes(const kda_desc* d, int32_t n_parts) {
  return align256((size_t)d->B * n_parts * d->H * d->d_k * d->d_v * sizeof(float));
}
}  // namespace

size_t kda_chunk_fwd_kcp_workspace_size(const kda_desc* d, int32_t n_parts) {
  if (validate_desc(d) != KDA_OK) return 0;
  if (n_parts == 1 || d->T == 0) return kda_chunk_fwd_workspace_size(d);
  kda_desc inner;
  if (head_first(d) || !kcp_shape(d, n_parts, &inner)) return 0;
  return 3 * kcp_state_bytes(d, n_parts) + kda_chunk_fwd_workspace_size(&inner);
}

kda_status kda_chunk_fwd_kcp(const kda_desc* d, int32_t n_parts, const void* q, const void* k, const void* v,
                             const void* beta, const void* z, const float* A, const float* S0, const void* gate,
                             const float* rms_w, void* o, void* y, float* S_T, void* ws, size_t ws_bytes,
                             void* stream) {
  kda_status st = validate_desc(d);
  if (st != KDA_OK) return st;
  if (n_parts < 1) return KDA_ERR_BAD_SHAPE;
  if (n_parts == 1 || d->T == 0)
    return chunk_fwd_impl(d, q, k, v, beta, z, A, S0, gate, rms_w, o, y, S_T, ws, ws_bytes, stream,
                          Tracer{nullptr, 0});
  kda_desc inner;
  // the segments are read as B * n_parts shorter sequences, which only the
  // token-major order lays out that way
  if (head_first(d) || !kcp_shape(d, n_parts, &inner)) return KDA_ERR_UNSUPPORTED;
  if (!o && !y && !S_T) return KDA_ERR_NULL_ARG;
  if (!q || !k || !v || !beta || !z || !A) return KDA_ERR_NULL_ARG;
  if (y && !gate) return KDA_ERR_NULL_ARG;
  if ((S0 && !aligned(S0, 4)) || (S_T && !aligned(S_T, 4))) return KDA_ERR_MISALIGNED;
  const size_t sb = kcp_state_bytes(d, n_parts);
  if (!ws || !aligned(ws, 16) || ws_bytes < 3 * sb) return KDA_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  float* M = reinterpret_cast<float*>(base);
  float* St = reinterpret_cast<float*>(base + sb);
  float* Sin = reinterpret_cast<float*>(base + 2 * sb);
  void* iws = base + 3 * sb;
  const size_t ibytes = ws_bytes - 3 * sb;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int D = d->d_k;
  const Tracer none{nullptr, 0};
  // pass 1: every segment's transfer (from the identity with V = 0) and its
  // state from zero, all segments at once
  st = check_launch(kda::launch_identity_states(M, (int64_t)inner.B * inner.H, D, s), s);
  if (st != KDA_OK) return st;
  st = chunk_fwd_impl(&inner, q, k, nullptr, beta, z, A, M, nullptr, nullptr, nullptr, nullptr, M, iws, ibytes, s,
                      none, Snapshots{nullptr, 1, 0}, true);
  if (st != KDA_OK) return st;
  st = chunk_fwd_impl(&inner, q, k, v, beta, z, A, nullptr, nullptr, nullptr, nullptr, nullptr, St, iws, ibytes, s,
                      none);
  if (st != KDA_OK) return st;
  // fold along each sequence: the entry state of every segment
  st = check_launch(kda::launch_kcp_fold(M, St, S0, Sin, d->B, n_parts, d->H, D, s), s);
  if (st != KDA_OK) return st;
  // pass 2: every segment from its entry state, with outputs; final states in place
  st = chunk_fwd_impl(&inner, q, k, v, beta, z, A, Sin, gate, rms_w, o, y, Sin, iws, ibytes, s, none);
  if (st != KDA_OK) return st;
  if (S_T) {
    const int64_t per = (int64_t)d->H * D * D;
    for (int b = 0; b < d->B; ++b) {
      st = check_launch(
          kda::launch_copy_state(Sin + ((int64_t)b * n_parts + n_parts - 1) * per, S_T + b * per, per, s), s);
      if (st != KDA_OK) return st;
    }
  }
  return KDA_OK;
}

int32_t kda_snapshot_count(const kda_desc* d, int32_t every_chunks) {
  if (validate_desc(d) != KDA_OK || every_chunks < 1) return 0;
  return d->T / (kChunk * every_chunks);
}

kda_status kda_recurrent_step(const kda_desc* d, const void* q, const void* k, const void* v, const void* beta,
                              const void* z, const float* A, float* S_pool, int32_t n_slots, const int32_t* slot,
                              const void* gate, const float* rms_w, void* o, void* y, uint32_t* status,
                              void* stream) {
  kda_status st = validate_desc(d);
  if (st != KDA_OK) return st;
  if (d->T != 1 || n_slots < 1 || (slot == nullptr && d->B > n_slots)) return KDA_ERR_BAD_SHAPE;
  if (!q || !k || !v || !beta || !z || !A || !S_pool) return KDA_ERR_NULL_ARG;
  if (!o && !y) return KDA_ERR_NULL_ARG;
  if (y && !gate) return KDA_ERR_NULL_ARG;
  const size_t es = elem_size(d->in_dtype);
  for (const void* p : {q, k, v, z, (const void*)o, (const void*)y, gate})
    if (p && !aligned(p, 16)) return KDA_ERR_MISALIGNED;
  if (!aligned(beta, es) || !aligned(A, 4) || !aligned(S_pool, 4) || (slot && !aligned(slot, 4)) ||
      (rms_w && !aligned(rms_w, 4)) || (status && !aligned(status, 4)))
    return KDA_ERR_MISALIGNED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  kda::DecodeParams p{};
  p.n_slots = n_slots;
  p.status = status;
  p.q = q;
  p.k = k;
  p.v = v;
  p.beta = beta;
  p.z = z;
  p.A = A;
  p.S_pool = S_pool;
  p.slot = slot;
  p.gate = y ? gate : nullptr;
  p.rms_w = rms_w;
  p.o = o;
  p.y = y;
  p.n = d->B;
  p.H = d->H;
  p.g_min = d->g_min;
  p.q_scale = d->q_scale;
  p.l2_eps = d->l2_eps;
  p.rms_eps = d->rms_eps;
  p.l2norm = d->qk_l2norm;
  p.decay = d->decay;
  p.out_f32 = d->out_dtype == KDA_F32;
  return check_launch(kda::launch_decode(p, d->d_k, d->in_dtype == KDA_F32, s), s);
}

kda_status kda_state_io(kda_state_op op, int32_t n, int32_t H, int32_t d_k, int32_t d_v, kda_state_layout layout,
                        float* pool, int32_t n_slots, const int32_t* slot, float* user, uint32_t* status,
                        void* stream) {
  const int op_i = enum_int(op), layout_i = enum_int(layout);
  if (op_i != KDA_STATE_ZERO && op_i != KDA_STATE_IMPORT && op_i != KDA_STATE_EXPORT) return KDA_ERR_UNSUPPORTED;
  if (layout_i != KDA_LAYOUT_KV && layout_i != KDA_LAYOUT_VK) return KDA_ERR_UNSUPPORTED;
  if (n < 0 || H < 1 || d_k < 1 || d_v < 1 || n_slots < 1 || (slot == nullptr && n > n_slots))
    return KDA_ERR_BAD_SHAPE;
  if (d_k != d_v || (d_k != 64 && d_k != 128)) return KDA_ERR_UNSUPPORTED;
  if (!pool) return KDA_ERR_NULL_ARG;
  if (op != KDA_STATE_ZERO && !user) return KDA_ERR_NULL_ARG;
  if (!aligned(pool, 4) || (user && !aligned(user, 4)) || (slot && !aligned(slot, 4)) || (status && !aligned(status, 4)))
    return KDA_ERR_MISALIGNED;
  if (n == 0) return KDA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  kda::StateIoParams p{};
  p.n_slots = n_slots;
  p.status = status;
  p.op = static_cast<int>(op);
  p.transpose = layout == KDA_LAYOUT_VK;
  p.n = n;
  p.H = H;
  p.pool = pool;
  p.slot = slot;
  p.user = user;
  p.vec16 = aligned(pool, 16) && (user == nullptr || aligned(user, 16));
  return check_launch(kda::launch_state_io(p, d_k, s), s);
}

kda_status kda_prepass(const kda_desc* d, const void* q, const void* k, const void* z, const float* A, float* G,
                       float* rq, float* rk, void* stream) {
  kda_status st = validate_desc(d);
  if (st != KDA_OK) return st;
  if (head_first(d)) return KDA_ERR_UNSUPPORTED;  // token major only
  if (!q || !k || !z || !A || !G || !rq || !rk) return KDA_ERR_NULL_ARG;
  for (const void* p : {q, k, z})
    if (!aligned(p, 16)) return KDA_ERR_MISALIGNED;
  if (!aligned(A, 4) || !aligned(G, 4) || !aligned(rq, 4) || !aligned(rk, 4)) return KDA_ERR_MISALIGNED;
  if (d->T == 0) return KDA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  kda::PrepassParams p{};
  p.q = q;
  p.k = k;
  p.z = z;
  p.A = A;
  p.B = d->B;
  p.T = d->T;
  p.H = d->H;
  p.g_min = d->g_min;
  p.l2_eps = d->l2_eps;
  p.l2norm = d->qk_l2norm;
  p.decay = d->decay;
  p.G = G;
  p.rq = rq;
  p.rk = rk;
  return check_launch(kda::launch_prepass(p, d->d_k, d->in_dtype == KDA_F32, s), s);
}

}  // extern "C"
