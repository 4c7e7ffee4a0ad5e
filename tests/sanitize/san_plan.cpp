// Driver for the AddressSanitizer / UndefinedBehaviorSanitizer build of the
// library's host layer: it includes kda_api.cpp itself, so that the internal
// planning steps (descriptor validation, pipelined_segments, layout_for,
// make_plan, plan_launches) can be called directly and their invariants
// checked over a sweep of shapes, and then drives the C ABI's queries and
// argument checks (every call here returns before any GPU work; no GPU is
// needed).  Built and run by tests/test_sanitizers.py; a sanitizer finding
// aborts it.
#include "kda_api.cpp"

#include <cstdio>

static int failures = 0;
#define EXPECT(c)                                                                        \
  do {                                                                                   \
    if (!(c)) {                                                                          \
      std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #c); \
      ++failures;                                                                        \
    }                                                                                    \
  } while (0)

static kda_desc make(int B, int T, int H, int D, kda_dtype dt, int seg, int overlap, int fused) {
  kda_desc d{};
  EXPECT(kda_desc_init(&d, B, T, H, D, dt, dt) == KDA_OK);
  d.segment_tokens = seg;
  d.overlap = overlap;
  d.fused = fused;
  return d;
}

static void check_segments(const kda_desc* d) {
  const int64_t nc = num_chunks(d);
  const int64_t len = pipelined_chunks(d);
  EXPECT(len >= 1);
  const int n = pipelined_segments(d, len);
  // no segment for an empty sequence; at most one per chunk (the counters the layout holds)
  EXPECT(n >= (nc > 0 ? 1 : 0) && n <= nc);
  if (n > 0) EXPECT((int64_t)(n - 1) * len < nc && (int64_t)n * len >= nc);  // they cover the chunks exactly
}

static void check_layout(const kda_desc* d, int64_t seg_nc) {
  const WsLayout L = layout_for(d, seg_nc);
  const size_t recs = (size_t)d->B * d->H * seg_nc * L.rec_bytes;
  EXPECT(L.off_rec % 256 == 0 && L.off_carry % 256 == 0 && L.off_done % 256 == 0);
  EXPECT(L.off_rec + recs <= L.off_carry);
  EXPECT(L.off_carry + (size_t)d->B * d->H * d->d_k * d->d_v * 4 <= L.off_done);
  EXPECT(L.off_done + (kStatusWords + (num_chunks(d) + 1) * (size_t)d->B * d->H) * 4 <= L.total);
  EXPECT(L.rec_bytes == (size_t)kda::rec_units((int)elem_size(d->in_dtype), d->d_k).bytes);
}

// the pipelined schedule's window for a workspace: none, the whole sequence,
// or the largest run of whole segments (at least kMinPipelinedWindow chunks)
// whose records fit
static void check_window(const kda_desc* d, size_t ws) {
  const int64_t nc = num_chunks(d), seg = pipelined_chunks(d);
  const int64_t w = pipelined_window(d, ws);
  EXPECT(w == 0 || w == nc || (w % seg == 0 && w >= kMinPipelinedWindow && w < nc));
  if (w > 0) EXPECT(layout_for(d, w).total <= ws);
  if (w > 0 && w < nc) EXPECT(layout_for(d, w + seg).total > ws);
}

static void check_plan(const kda_desc* d, size_t ws_bytes) {
  const Plan p = make_plan(d, ws_bytes);
  const int64_t nc = num_chunks(d);
  EXPECT(p.seg_nc >= 1);
  EXPECT(!(p.fused && p.pipelined) && !(p.overlapped && p.pipelined));
  if (p.pipelined) {  // windows: the whole sequence or whole segments that fit
    EXPECT(p.window >= 1 && p.window <= (nc < 1 ? 1 : nc));
    EXPECT(p.window == nc || (p.window % p.seg_nc == 0 && p.window >= kMinPipelinedWindow));
    EXPECT(layout_for(d, p.window).total <= ws_bytes);
  }
  if (!p.fused && !p.pipelined && !p.overlapped && ws_bytes >= layout_for(d, 1).total) {
    EXPECT(layout_for(d, p.seg_nc).total <= ws_bytes);  // the chosen segment fits
    EXPECT(p.seg_nc <= (nc < 1 ? 1 : nc));
  }
  int32_t kinds[4096];
  const int32_t n = plan_launches(d, p, kinds, 4096);
  EXPECT(n >= (nc > 0 || p.fused ? 1 : 0));
  const int32_t m = plan_launches(d, p, nullptr, 0);  // the count alone
  EXPECT(m == n);
}

alignas(256) static char buf[4096];

int main() {
  // internal planning over a sweep of shapes
  const int Ts[] = {0, 1, 63, 64, 65, 130, 4096, 4097, 65536, 65536 * 3 + 17, 1 << 20};
  const int segs[] = {0, 64, 100, 512, 4096, 8192, 65536};
  for (kda_dtype dt : {KDA_BF16, KDA_F32})
    for (int D : {64, 128})
      for (int T : Ts)
        for (int seg : segs)
          for (int ov : {0, 1}) {
            kda_desc d = make(2, T, 3, D, dt, seg, ov, 1);
            EXPECT(validate_desc(&d) == KDA_OK);
            check_segments(&d);
            for (int64_t sn : {int64_t(1), int64_t(7), num_chunks(&d) < 1 ? int64_t(1) : num_chunks(&d)})
              check_layout(&d, sn);
            for (size_t ws : {size_t(0), layout_for(&d, 1).total, layout_for(&d, 3).total - 1,
                              layout_for(&d, 700).total, layout_for(&d, 2049).total + 100,
                              kda_chunk_fwd_workspace_size(&d), size_t(1) << 40})
            {
              check_plan(&d, ws);
              check_window(&d, ws);
            }
          }
  // the fused schedule on request (bf16, K3 decay): one launch, no workspace
  for (int T : Ts) {
    kda_desc f = make(1, T, 4, 128, KDA_BF16, 0, 1, 2);
    check_plan(&f, 0);
    EXPECT(make_plan(&f, 0).fused);
  }
  // descriptor validation
  kda_desc d = make(1, 128, 2, 128, KDA_BF16, 0, 1, 1);
  EXPECT(validate_desc(nullptr) == KDA_ERR_NULL_ARG);
  kda_desc bad = d;
  bad.d_k = 96;
  bad.d_v = 96;
  EXPECT(validate_desc(&bad) == KDA_ERR_UNSUPPORTED);
  bad = d;
  bad.T = -1;
  EXPECT(validate_desc(&bad) == KDA_ERR_BAD_SHAPE);
  bad = d;
  const int seven = 7;  // an int a C caller may store in the enum field
  std::memcpy(&bad.in_dtype, &seven, sizeof seven);
  EXPECT(validate_desc(&bad) == KDA_ERR_BAD_DTYPE);
  bad = d;
  std::memcpy(&bad.decay, &seven, sizeof seven);
  EXPECT(validate_desc(&bad) == KDA_ERR_UNSUPPORTED);
  EXPECT(kda_state_io(KDA_STATE_IMPORT, 1, 1, 128, 128, KDA_LAYOUT_KV, reinterpret_cast<float*>(buf), 1, nullptr,
                      nullptr, nullptr, nullptr) == KDA_ERR_NULL_ARG);  // import without the caller's states
  bad = d;
  bad.g_min = 1.0f;
  EXPECT(validate_desc(&bad) == KDA_ERR_UNSUPPORTED);
  bad = d;
  bad.fused = 3;
  EXPECT(validate_desc(&bad) == KDA_ERR_BAD_SHAPE);
  bad = d;
  std::memcpy(&bad.tokens, &seven, sizeof seven);
  EXPECT(validate_desc(&bad) == KDA_ERR_UNSUPPORTED);
  bad = d;
  bad.tokens = KDA_TOKENS_BHTD;
  EXPECT(validate_desc(&bad) == KDA_OK && head_first(&bad) == 1 && head_first(&d) == 0);
  EXPECT(kda_desc_init(nullptr, 1, 1, 1, 128, KDA_BF16, KDA_BF16) == KDA_ERR_NULL_ARG);

  // C ABI queries and argument checks (all return before any GPU work)
  EXPECT(kda_abi_version() == KDA_ABI_VERSION);
  for (int s = 0; s <= 9; ++s) EXPECT(kda_status_str((kda_status)s) != nullptr);
  int32_t seg = 0, sched = -1, kinds[8], n_launch = 0;
  EXPECT(kda_chunk_fwd_schedule(&d, kda_chunk_fwd_workspace_size(&d), &seg, &sched) == KDA_OK);
  EXPECT(kda_chunk_fwd_launches(&d, kda_chunk_fwd_workspace_size(&d), kinds, 8, &n_launch) == KDA_OK && n_launch >= 1);
  EXPECT(kda_chunk_fwd_workspace_size(nullptr) == 0);
  EXPECT(kda_snapshot_count(&d, 0) <= 0 && kda_snapshot_count(&d, 1) == 2);
  char* mis = buf + 2;  // misaligned
  EXPECT(kda_chunk_fwd(&d, nullptr, buf, buf, buf, buf, (const float*)buf, nullptr, nullptr, nullptr, buf, nullptr,
                       nullptr, buf, sizeof(buf), nullptr) == KDA_ERR_NULL_ARG);
  EXPECT(kda_chunk_fwd(&d, mis, buf, buf, buf, buf, (const float*)buf, nullptr, nullptr, nullptr, buf, nullptr, nullptr,
                       buf, sizeof(buf), nullptr) == KDA_ERR_MISALIGNED);
  EXPECT(kda_chunk_fwd(&bad, buf, buf, buf, buf, buf, (const float*)buf, nullptr, nullptr, nullptr, buf, nullptr,
                       nullptr, buf, sizeof(buf), nullptr) != KDA_OK);
  EXPECT(kda_chunk_fwd(&d, buf, buf, buf, buf, buf, (const float*)buf, nullptr, nullptr, nullptr, buf, buf, nullptr,
                       buf, sizeof(buf), nullptr) == KDA_ERR_NULL_ARG);  // y without the gate
  if (failures) {
    std::fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  std::printf("san_plan: ok\n");
  return 0;
}
