// Host driver for the sanitizer build of the C ABI's argument validation
// (include/kda.h, kda_api.cpp) with the kernel launchers stubbed out (test
// infrastructure).  Fake, never dereferenced device pointers go through every
// entry point, valid and invalid; a valid call must reach its launcher with
// the sizes it was given, an invalid one must return its status without
// launching.  Exit status 0 means every check held.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kda.h"
#include "launch_stubs.h"

static int fails = 0;
#define CHECK(c, ...) do { if (!(c)) { fprintf(stderr, __VA_ARGS__); fputc('\n', stderr); ++fails; } } while (0)

static void* P = reinterpret_cast<void*>(uintptr_t(4096));  // aligned fake address
static float* F = reinterpret_cast<float*>(uintptr_t(4096));
static void* P2 = reinterpret_cast<void*>(uintptr_t(4096 + 2));

template <class Fn>
static void expect(const char* what, kda_status want, bool launches, Fn call) {
  const int before = g_last.count;
  const kda_status got = call();
  CHECK(got == want, "%s: status %d (%s), expected %d", what, (int)got, kda_status_string(got),
        (int)want);
  CHECK((g_last.count > before) == launches, "%s: launched %d", what, g_last.count - before);
}

int main() {
  for (int s = 0; s <= 6; ++s) CHECK(kda_status_string((kda_status)s) != nullptr, "status string");
  CHECK(strcmp(kda_status_string((kda_status)99), "unknown kda_status") == 0, "unknown status");
  CHECK(kda_version() >= 10000, "version");

  // kda_gate
  expect("gate ok", KDA_OK, true, [] {
    return kda_gate(F, F, F, KDA_GATE_SAFE, -5.f, 2, 64, 4, 128, 64, F, nullptr); });
  expect("gate L>=0", KDA_ERR_INVALID_ARG, false, [] {
    return kda_gate(F, F, F, KDA_GATE_SAFE, 1.f, 2, 64, 4, 128, 0, F, nullptr); });
  expect("gate empty", KDA_OK, false, [] {
    return kda_gate(F, F, F, KDA_GATE_SAFE, -5.f, 0, 64, 4, 128, 0, F, nullptr); });
  expect("gate kind", KDA_ERR_INVALID_ARG, false, [] {
    return kda_gate(F, F, F, (kda_gate_kind)9, -5.f, 1, 1, 1, 1, 0, F, nullptr); });

  // kda_chunk_fwd
  auto chunk = [](int B, int T, int H, int HV, int K, int V, int C, const void* q, float L) {
    return kda_chunk_fwd(q, P, P, KDA_BF16, F, F, F, F, KDA_GATE_SAFE, L, nullptr, F, F, B, T, H,
                         HV, K, V, C, nullptr, 0, nullptr);
  };
  expect("chunk ok", KDA_OK, true, [&] { return chunk(2, 100, 2, 8, 128, 128, 64, P, -5.f); });
  CHECK(g_last.B == 2 && g_last.T == 100 && g_last.H == 2 && g_last.HV == 8 && g_last.K == 128,
        "chunk sizes not forwarded");
  expect("chunk HV%H", KDA_ERR_INVALID_ARG, false, [&] { return chunk(1, 64, 3, 8, 128, 128, 64, P, -5.f); });
  expect("chunk K", KDA_ERR_UNSUPPORTED, false, [&] { return chunk(1, 64, 2, 8, 96, 96, 64, P, -5.f); });
  expect("chunk C", KDA_ERR_UNSUPPORTED, false, [&] { return chunk(1, 64, 2, 8, 128, 128, 48, P, -5.f); });
  expect("chunk align", KDA_ERR_INVALID_ARG, false, [&] { return chunk(1, 64, 2, 8, 128, 128, 64, P2, -5.f); });
  expect("chunk null", KDA_ERR_INVALID_ARG, false, [&] { return chunk(1, 64, 2, 8, 128, 128, 64, nullptr, -5.f); });
  expect("chunk B=0", KDA_OK, false, [&] { return chunk(0, 64, 2, 8, 128, 128, 64, P, -5.f); });
  expect("chunk T<0", KDA_ERR_INVALID_ARG, false, [&] { return chunk(1, -1, 2, 8, 128, 128, 64, P, -5.f); });
  expect("chunk wide", KDA_ERR_UNSUPPORTED, false, [&] { return chunk(1, 64, 1, 1 << 18, 128, 128, 64, P, -5.f); });

  // kda_recurrent_step / kda_recurrent_fwd
  expect("step ok", KDA_OK, true, [] {
    return kda_recurrent_step(P, P, P, KDA_F32, F, F, F, F, KDA_GATE_STANDARD, -5.f, F, F, 4, 2, 4,
                              64, 32, nullptr); });
  expect("step V", KDA_ERR_UNSUPPORTED, false, [] {
    return kda_recurrent_step(P, P, P, KDA_F32, F, F, F, F, KDA_GATE_STANDARD, -5.f, F, F, 4, 2, 4,
                              64, 48, nullptr); });
  expect("rec ok", KDA_OK, true, [] {
    return kda_recurrent_fwd(P, P, P, KDA_BF16, F, F, F, F, KDA_GATE_NONE, 0.f, nullptr, F, F, 1,
                             7, 1, 2, 16, 128, nullptr); });
  expect("rec A_log", KDA_ERR_INVALID_ARG, false, [] {
    return kda_recurrent_fwd(P, P, P, KDA_BF16, F, F, nullptr, F, KDA_GATE_SAFE, -5.f, nullptr, F,
                             F, 1, 7, 1, 2, 16, 128, nullptr); });

  // kda_chunk_fwd_split and its allocation-free variant
  const size_t need = kda_chunk_fwd_split_workspace_bytes(1, 100, 2, 4, 128, 128, 64);
  CHECK(need > 0, "split workspace size");
  expect("split ok", KDA_OK, true, [&] {
    return kda_chunk_fwd_split(P, P, P, KDA_BF16, F, F, F, F, KDA_GATE_SAFE, -5.f, nullptr, F, F,
                               nullptr, 1, 100, 2, 4, 128, 128, 64, P, need, nullptr); });
  CHECK(g_last.workspace == P, "split workspace not forwarded");
  expect("split small ws", KDA_ERR_WORKSPACE, false, [&] {
    return kda_chunk_fwd_split(P, P, P, KDA_BF16, F, F, F, F, KDA_GATE_SAFE, -5.f, nullptr, F, F,
                               nullptr, 1, 100, 2, 4, 128, 128, 64, P, need - 1, nullptr); });
  expect("split states only", KDA_OK, true, [&] {
    return kda_chunk_fwd_split(P, P, P, KDA_BF16, F, F, F, F, KDA_GATE_SAFE, -5.f, nullptr,
                               nullptr, nullptr, F, 1, 100, 2, 4, 128, 128, 64, P, need, nullptr); });
  expect("split no o, no h", KDA_ERR_INVALID_ARG, false, [&] {
    return kda_chunk_fwd_split(P, P, P, KDA_BF16, F, F, F, F, KDA_GATE_SAFE, -5.f, nullptr,
                               nullptr, F, nullptr, 1, 100, 2, 4, 128, 128, 64, P, need, nullptr); });
  expect("noalloc ok", KDA_OK, true, [&] {
    return kda_chunk_fwd_split_noalloc(P, P, P, KDA_BF16, F, F, F, F, KDA_GATE_SAFE, -5.f, nullptr,
                                       F, F, nullptr, 1, 100, 2, 4, 128, 128, 64, nullptr); });
  CHECK(g_last.workspace != nullptr && g_last.workspace != P, "noalloc scratch not used");
  expect("noalloc too big", KDA_ERR_SCRATCH, false, [&] {
    return kda_chunk_fwd_split_noalloc(P, P, P, KDA_BF16, F, F, F, F, KDA_GATE_SAFE, -5.f, nullptr,
                                       F, F, nullptr, 4, 65536, 16, 64, 128, 128, 64, nullptr); });

  // kda_bwd
  const size_t bneed = kda_bwd_workspace_bytes(2, 37, 2, 4, 64, 64);
  CHECK(bneed > 0, "bwd workspace size");
  CHECK(kda_bwd_workspace_bytes(2, 37, 2, 4, 16, 16) == 0, "bwd workspace of an unsupported size");
  auto bwd = [&](kda_gate_kind gate, int K, int V, const void* q, float* dq, void* ws, size_t wsb,
                 int H, int HV, int T) {
    return kda_bwd(q, P, P, KDA_F32, F, F, F, F, gate, -5.f, F, F, nullptr, dq, F, F, F, F, F, F,
                   F, 2, T, H, HV, K, V, ws, wsb, nullptr);
  };
  expect("bwd ok", KDA_OK, true, [&] { return bwd(KDA_GATE_SAFE, 64, 64, P, F, P, bneed, 2, 4, 37); });
  CHECK(g_last.B == 2 && g_last.T == 37 && g_last.H == 2 && g_last.HV == 4 && g_last.K == 64 &&
        g_last.workspace == P, "bwd sizes not forwarded");
  expect("bwd small ws", KDA_ERR_WORKSPACE, false, [&] {
    return bwd(KDA_GATE_SAFE, 64, 64, P, F, P, bneed - 1, 2, 4, 37); });
  expect("bwd per-head", KDA_OK, true, [&] {
    return bwd((kda_gate_kind)(KDA_GATE_SAFE | KDA_GATE_PER_HEAD), 64, 64, P, F, P, bneed, 2, 4, 37); });
  expect("bwd K=16", KDA_ERR_UNSUPPORTED, false, [&] { return bwd(KDA_GATE_SAFE, 16, 16, P, F, P, bneed, 2, 4, 37); });
  expect("bwd K!=V", KDA_ERR_UNSUPPORTED, false, [&] { return bwd(KDA_GATE_SAFE, 64, 32, P, F, P, bneed, 2, 4, 37); });
  expect("bwd null dq", KDA_ERR_INVALID_ARG, false, [&] { return bwd(KDA_GATE_SAFE, 64, 64, P, nullptr, P, bneed, 2, 4, 37); });
  expect("bwd align", KDA_ERR_INVALID_ARG, false, [&] { return bwd(KDA_GATE_SAFE, 64, 64, P2, F, P, bneed, 2, 4, 37); });
  expect("bwd HV%H", KDA_ERR_INVALID_ARG, false, [&] { return bwd(KDA_GATE_SAFE, 64, 64, P, F, P, bneed, 3, 4, 37); });
  expect("bwd T=0", KDA_OK, true, [&] { return bwd(KDA_GATE_SAFE, 64, 64, P, F, nullptr, 0, 2, 4, 0); });

  if (fails) { fprintf(stderr, "%d check(s) failed\n", fails); return 1; }
  printf("api driver: all checks passed (%d launches)\n", g_last.count);
  return 0;
}
