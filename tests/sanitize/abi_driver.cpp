// Exercises the host side of the C ABI -- the pure host helpers and the
// validation of every entry point -- for the AddressSanitizer and
// UndefinedBehaviorSanitizer build of the library's host code (test
// infrastructure).  Every compute call here is rejected before anything is
// enqueued (or has an empty batch), so no GPU is needed.  Exit status 0
// when every call returns the expected status.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "rat.h"

static int fails = 0;
static void expect(const char* what, int64_t got, int64_t want) {
  if (got != want) {
    std::printf("FAIL %s: got %lld, want %lld\n", what, (long long)got, (long long)want);
    ++fails;
  }
}

int main() {
  // fake device pointers: only passed to calls that validation rejects
  alignas(16) static char buf[4096];
  void* p = buf;
  void* mis = buf + 8;  // not 16-byte aligned
  float* fp = reinterpret_cast<float*>(buf);
  const int H = 3;
  const int32_t D[H] = {4, 1, 16}, W[H] = {0, 5, 3};
  const int32_t Dbad[H] = {4, 0, 16}, Wbad[H] = {0, -1, 3};

  expect("version", std::strlen(rat_version()) > 0, 1);
  for (int c = 1; c >= -6; --c) expect("status string", rat_status_string(c) != nullptr, 1);

  int64_t off[H + 1];
  expect("anchor rows", rat_anchor_rows(H, 100, D, off), 25 + 100 + 6);
  expect("anchor offsets", off[2], 125);
  expect("anchor rows, D = 0", rat_anchor_rows(H, 100, Dbad, nullptr), RAT_ERR_INVALID_ARG);
  expect("anchor rows, null D", rat_anchor_rows(H, 100, nullptr, nullptr), RAT_ERR_INVALID_ARG);
  expect("ring rows", rat_ring_rows(H, W, off), 8);
  expect("ring rows, W < 0", rat_ring_rows(H, Wbad, nullptr), RAT_ERR_INVALID_ARG);
  for (int64_t T : {0, 1, 63, 64, 65, 4097, 100000})
    for (int hd : {64, 128}) {
      const int64_t n = rat_scan_workspace_bytes(3, 5, T, hd);
      expect("scan workspace > 0", n > 0, 1);
    }
  expect("scan workspace, hd 96", rat_scan_workspace_bytes(1, 1, 10, 96), RAT_ERR_UNSUPPORTED);
  expect("scan workspace, T < 0", rat_scan_workspace_bytes(1, 1, -1, 64), RAT_ERR_INVALID_ARG);
  expect("decode workspace", rat_decode_workspace_bytes(2, H, 128, 1000, D, W, 4) > 0, 1);
  expect("decode workspace, 1 split", rat_decode_workspace_bytes(2, H, 128, 1000, D, W, 1), 0);
  expect("decode workspace, D = 0", rat_decode_workspace_bytes(2, H, 128, 1000, Dbad, W, 0),
         RAT_ERR_INVALID_ARG);
  expect("backward workspace", rat_prefill_backward_workspace_bytes(2, H, 300, 64, D, W) > 0, 1);
  expect("layer workspace", rat_layer_workspace_bytes(RAT_DTYPE_BF16, 2, H, 300, 64) > 0, 1);
  expect("layer workspace, dtype", rat_layer_workspace_bytes(9, 2, H, 300, 64),
         RAT_ERR_UNSUPPORTED);

  const size_t wsb = sizeof(buf);
  // scan: bad dtype, head dim, per-head tables, capacity, pointers, workspace
  expect("scan dtype", rat_scan_prefill(5, 1, H, 10, 64, D, W, 20, p, p, p, p, p, p, p, p, p, fp, fp,
                                        p, wsb, nullptr), RAT_ERR_UNSUPPORTED);
  expect("scan hd", rat_scan_prefill(0, 1, H, 10, 96, D, W, 20, p, p, p, p, p, p, p, p, p, fp, fp,
                                     p, wsb, nullptr), RAT_ERR_UNSUPPORTED);
  expect("scan D", rat_scan_prefill(0, 1, H, 10, 64, Dbad, W, 20, p, p, p, p, p, p, p, p, p, fp, fp,
                                    p, wsb, nullptr), RAT_ERR_INVALID_ARG);
  expect("scan capacity", rat_scan_prefill(0, 1, H, 30, 64, D, W, 20, p, p, p, p, p, p, p, p, p,
                                           fp, fp, p, wsb, nullptr), RAT_ERR_CAPACITY);
  expect("scan null k", rat_scan_prefill(0, 1, H, 10, 64, D, W, 20, nullptr, p, p, p, p, p, p, p, p,
                                         fp, fp, p, wsb, nullptr), RAT_ERR_INVALID_ARG);
  expect("scan misaligned", rat_scan_prefill(0, 1, H, 10, 64, D, W, 20, mis, p, p, p, p, p, p, p, p,
                                             fp, fp, p, wsb, nullptr), RAT_ERR_INVALID_ARG);
  expect("scan workspace", rat_scan_prefill(0, 1, H, 10, 64, D, W, 20, p, p, p, p, p, p, p, p, p,
                                            fp, fp, p, 16, nullptr), RAT_ERR_WORKSPACE);
  expect("scan empty batch", rat_scan_prefill(0, 0, H, 10, 64, D, W, 20, p, p, p, p, p, p, p, p, p,
                                              fp, fp, p, wsb, nullptr), RAT_OK);
  expect("continue, same state", rat_scan_prefill_continue(0, 1, H, 10, 64, D, W, 40, 5, p, p, p,
                                                           fp, fp, p, p, p, p, p, p, p, p, fp, fp,
                                                           p, wsb, nullptr), RAT_ERR_INVALID_ARG);
  // attention
  expect("attn scale", rat_dilated_attn_prefill(0, 1, H, 10, 64, D, W, 1.0f / 0.0f, 20, p, p, p, p,
                                                p, p, nullptr, nullptr), RAT_ERR_INVALID_ARG);
  expect("attn capacity", rat_dilated_attn_prefill(0, 1, H, 30, 64, D, W, 0.f, 20, p, p, p, p, p, p,
                                                   nullptr, nullptr), RAT_ERR_CAPACITY);
  expect("attn null o", rat_dilated_attn_prefill(0, 1, H, 10, 64, D, W, 0.f, 20, p, p, p, p, p,
                                                 nullptr, nullptr, nullptr), RAT_ERR_INVALID_ARG);
  expect("attn continue ring", rat_dilated_attn_prefill_continue(0, 1, H, 10, 64, D, W, 0.f, 40, 5,
                                                                 p, p, p, p, p, nullptr, nullptr, p,
                                                                 nullptr, nullptr),
         RAT_ERR_INVALID_ARG);
  // decode
  expect("decode capacity", rat_decode_step(0, 1, H, 64, D, W, 0.f, 20, 20, p, p, p, p, fp, fp, p,
                                            p, p, p, p, 0, p, wsb, nullptr), RAT_ERR_CAPACITY);
  expect("decode splits", rat_decode_step(0, 1, H, 64, D, W, 0.f, 5, 20, p, p, p, p, fp, fp, p, p,
                                          p, p, p, 2000, p, wsb, nullptr), RAT_ERR_INVALID_ARG);
  expect("decode workspace", rat_decode_step(0, 1, H, 64, D, W, 0.f, 5, 1000, p, p, p, p, fp, fp, p,
                                             p, p, p, p, 8, nullptr, 0, nullptr),
         RAT_ERR_WORKSPACE);
  expect("decode misaligned", rat_decode_step(0, 1, H, 64, D, W, 0.f, 5, 20, mis, p, p, p, fp, fp,
                                              p, p, p, p, p, 0, p, wsb, nullptr),
         RAT_ERR_INVALID_ARG);
  // top-k decode and its history build
  expect("topk k", rat_decode_step_topk(0, 1, H, 64, D, W, 0.f, 5, 200, RAT_TOPK_MAX_K + 1, p, p, p,
                                        p, fp, fp, p, p, p, p, p, p, fp, p, nullptr, nullptr),
         RAT_ERR_UNSUPPORTED);
  expect("topk build capacity", rat_topk_cache_build(0, 1, H, 30, 64, 20, 0, p, p, p, p, fp,
                                                     nullptr), RAT_ERR_CAPACITY);
  // backward and layer
  expect("backward workspace", rat_prefill_backward(0, 1, H, 10, 64, D, W, 0.f, p, p, p, p, p, p, p,
                                                    fp, p, p, p, p, p, p, 16, nullptr),
         RAT_ERR_WORKSPACE);
  expect("backward null dO", rat_prefill_backward(0, 1, H, 10, 64, D, W, 0.f, p, p, p, p, p, p, p,
                                                  fp, nullptr, p, p, p, p, p, wsb, nullptr),
         RAT_ERR_INVALID_ARG);
  expect("layer dm", rat_layer_prefill(0, 1, H, 10, 64, 0, D, W, 0.f, 20, p, p, p, p, p, fp, p, p,
                                       fp, p, p, p, p, fp, fp, p, wsb, nullptr),
         RAT_ERR_INVALID_ARG);
  expect("layer workspace", rat_layer_prefill(0, 1, H, 10, 64, 64, D, W, 0.f, 20, p, p, p, p, p, fp,
                                              p, p, fp, p, p, p, p, fp, fp, p, 16, nullptr),
         RAT_ERR_WORKSPACE);

  std::printf("abi driver: %s (%d failures)\n", fails ? "FAILED" : "ok", fails);
  return fails ? 1 : 0;
}
