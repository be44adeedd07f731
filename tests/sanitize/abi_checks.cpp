// Host sanitizer run of the C ABI's host code (test infrastructure): the real
// argument checks and workspace layout of moe_api.cpp and the miss-policy
// replay of miss_replay.cpp, built with -fsanitize=address,undefined. Kernel
// launchers are replaced by stubs that abort, so every call here must be
// rejected on the host before any launch. Exit 0 and "ok" on success.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "kernels.hpp"
#include "moe.h"

#define CHECK(c)                                                              \
  do {                                                                        \
    if (!(c)) {                                                               \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);   \
      std::exit(1);                                                           \
    }                                                                         \
  } while (0)

namespace moe {
[[noreturn]] static void launched(const char* what) {
  std::fprintf(stderr, "a host check let %s launch\n", what);
  std::abort();
}
hipError_t launch_logits(const void*, int, int, int, const float*, int, float*, int*, bool, hipStream_t,
                         int64_t) { launched("router logits"); }
hipError_t launch_topk(const float*, int, int, int, int, int, int32_t*, float*, int32_t*, float*, hipStream_t) {
  launched("top-k");
}
hipError_t launch_group(const int32_t*, int, int, int, const GroupBufs&, hipStream_t) { launched("grouping"); }
hipError_t launch_decode_t1(const void*, int, const ExpertsDev&, int, int, const float*, const int32_t*, const float*,
                            int32_t*, float*, int32_t*, float*, float*, float*, bool, hipStream_t) {
  launched("single-token decode");
}
hipError_t launch_stage_experts(const ExpertsDev&, const ExpertsDev&, const int32_t*, const int32_t*, int,
                                hipStream_t) { launched("staging"); }
hipError_t launch_remap_ids(const int32_t*, int64_t, const int32_t*, int, int32_t*, hipStream_t) { launched("remap"); }
hipError_t launch_stream_read(const void*, int64_t, hipStream_t) { launched("stream read"); }
hipError_t launch_decode_grouped(const void*, int, int, const ExpertsDev&, int, const GroupBufs&, const float*, float*,
                                 float*, float*, hipStream_t) { launched("grouped decode"); }
hipError_t launch_combine(int, int, int, const float*, const float*, const uint16_t*, const int32_t*, float*, hipStream_t) {
  launched("combine");
}
hipError_t launch_gemm_grouped(const void*, int, int, const ExpertsDev&, int, const GroupBufs&, const float*,
                               uint16_t*, int32_t*, float*, float*, hipStream_t) { launched("grouped GEMM"); }
hipError_t launch_prerouter(const void*, int, int, const HeadDev&, const int32_t*, const int32_t*, int, int, float*,
                            float*, float*, int32_t*, float*, float*, hipStream_t) { launched("prerouter"); }
hipError_t launch_qlinear_lora(const void*, int, int, int, int, int, const uint8_t*, const uint16_t*, const float*,
                               const float*, int, float, float*, float*, hipStream_t) { launched("LoRA linear"); }
bool prerouted_t1_fusable(const ExpertsDev&, int, const HeadDev&) { return false; }
hipError_t launch_prerouted_t1(const void*, int, const ExpertsDev&, int, int, const float*, int32_t*, float*,
                               int32_t*, float*, float*, float*, const HeadDev&, const int32_t*, float*, float*,
                               float*, hipStream_t) { launched("prerouted decode"); }
hipError_t launch_quantize(const float*, int64_t, int, int, uint8_t*, uint16_t*, hipStream_t) {
  launched("quantiser");
}
}  // namespace moe

static void* const F = reinterpret_cast<void*>(0x10000);          // aligned, never dereferenced
static void* const MIS = reinterpret_cast<void*>(0x10008);        // misaligned
static float* const FF = reinterpret_cast<float*>(0x10000);
static int32_t* const FI = reinterpret_cast<int32_t*>(0x10000);
static uint16_t* const FS = reinterpret_cast<uint16_t*>(0x10000);

static moe_experts experts(int32_t E, int32_t H, int32_t I, int32_t scheme, const void* w = F) {
  return moe_experts{E, H, I, scheme, w, FS, F, FS};
}

static void rejected(moe_status st) {
  CHECK(st != MOE_OK);
  CHECK(std::strlen(moe_last_error()) > 0);
  CHECK(std::strlen(moe_status_str(st)) > 0);
}

int main() {
  // workspace sizes over the limits' corners
  const int32_t Ts[] = {0, 1, 2, 63, 64, 65, 127, 128, 2048, 65536, 65537};
  const int32_t Es[] = {0, 1, 16, 256, 1024, 1025};
  const int32_t Hs[] = {16, 32, 96, 4096, 4128};
  const int32_t ks[] = {0, 1, 8, 16, 17};
  for (int32_t T : Ts)
    for (int32_t E : Es)
      for (int32_t H : Hs)
        for (int32_t k : ks)
          for (int32_t s = 0; s < 3; ++s) {
            const size_t n = moe_workspace_bytes(T, E, H, H, k, s);
            const bool ok = T >= 1 && T <= 65536 && E >= 1 && E <= 1024 && H >= 32 && H <= 4096 && k >= 1 &&
                            k <= 16 && k <= E && s < 2;
            CHECK((n > 0) == ok);
            CHECK(n % 256 == 0);
          }
  CHECK(moe_prerouter_workspace_bytes(1, 256, 256) > 0 && moe_prerouter_workspace_bytes(1, 3, 256) == 0);
  CHECK(moe_qlinear_lora_workspace_bytes(1, 16) > 0 && moe_qlinear_lora_workspace_bytes(1, 65) == 0);

  const moe_experts ex = experts(256, 2048, 512, MOE_Q_SYM8);
  const moe_experts bad_codec = experts(256, 2048, 512, 5);
  const moe_experts bad_h = experts(256, 2000, 512, MOE_Q_SYM8);
  const moe_experts null_w = experts(256, 2048, 512, MOE_Q_SYM8, nullptr);
  const size_t big = (size_t)1 << 40;
  // router
  rejected(moe_route(nullptr, MOE_F16, 1, 2048, FF, 256, 8, 1, FI, FF, F, big, nullptr));
  rejected(moe_route(F, 9, 1, 2048, FF, 256, 8, 1, FI, FF, F, big, nullptr));
  rejected(moe_route(F, MOE_F16, 1, 2048, FF, 256, 8, 1, FI, FF, F, 16, nullptr));
  rejected(moe_route(F, MOE_F16, 1, 2048, FF, 256, 8, 1, FI, FF, MIS, big, nullptr));
  // grouping
  rejected(moe_group(FI, 1, 8, 256, nullptr, FI, FI, FI, FI, F, big, nullptr));
  rejected(moe_group(FI, 1, 8, 256, FI, FI, FI, FI, FI, F, 8, nullptr));
  // gathered experts and the layer
  rejected(moe_gather_qmm_forward(F, MOE_F16, 1, &bad_codec, 8, FI, FF, FF, 0, F, big, nullptr));
  rejected(moe_gather_qmm_forward(F, MOE_F16, 1, &bad_h, 8, FI, FF, FF, 0, F, big, nullptr));
  rejected(moe_gather_qmm_forward(F, MOE_F16, 1, &null_w, 8, FI, FF, FF, 0, F, big, nullptr));
  rejected(moe_gather_qmm_forward(F, MOE_F32, 4, &ex, 8, FI, FF, FF, MOE_FLAG_PATH_GEMM, F, big, nullptr));
  rejected(moe_gather_qmm_forward(F, MOE_F16, 4, &ex, 8, FI, FF, FF, 6, F, big, nullptr));
  rejected(moe_layer_forward(F, MOE_F16, 1, nullptr, &ex, 8, 1, FF, nullptr, nullptr, F, big, nullptr));
  rejected(moe_layer_forward(F, MOE_F16, 1, FF, &ex, 300, 1, FF, nullptr, nullptr, F, big, nullptr));
  rejected(moe_layer_forward(F, MOE_F16, 70000, FF, &ex, 8, 1, FF, nullptr, nullptr, F, big, nullptr));
  rejected(moe_layer_forward_noalloc(F, MOE_BF16, 2048, FF, &ex, 8, 1, FF, nullptr, nullptr, nullptr));
  const moe_experts stack8 = experts(8, 2048, 512, MOE_Q_SYM8);
  rejected(moe_layer_forward_staged(F, MOE_F16, 1, FF, 256, nullptr, FI, 8, 1, FF, nullptr, nullptr, F, big, nullptr));
  rejected(moe_layer_forward_staged(F, MOE_F16, 1, FF, 256, &stack8, nullptr, 8, 1, FF, nullptr, nullptr, F, big,
                                    nullptr));
  rejected(moe_layer_forward_staged(F, MOE_F16, 1, FF, 2000, &stack8, FI, 8, 1, FF, nullptr, nullptr, F, big,
                                    nullptr));
  rejected(moe_layer_forward_staged(F, MOE_F16, 1, FF, 256, &stack8, FI, 8, 1, FF, nullptr, nullptr, F, 64, nullptr));
  rejected(moe_layer_forward_noalloc(F, MOE_F16, 1, FF, &ex, 8, 0x40, FF, nullptr, nullptr, nullptr));
  rejected(moe_experts_from_logits(F, MOE_F16, 1, nullptr, &ex, 8, 1, FF, nullptr, nullptr, F, big, nullptr));
  rejected(moe_experts_from_logits(F, MOE_F16, 1, reinterpret_cast<float*>(MIS), &ex, 8, 1, FF, nullptr, nullptr, F,
                                   big, nullptr));
  // prerouter, prerouted layer
  moe_prerouter head{2048, 256, 256, FF, nullptr, FF, nullptr, FF};
  moe_prerouter odd_e{2048, 255, 256, FF, nullptr, FF, nullptr, FF};
  rejected(moe_prerouter_forward(F, MOE_F16, 1, &odd_e, nullptr, nullptr, 8, 1, FI, FF, nullptr, F, big, nullptr));
  rejected(moe_prerouter_forward(F, MOE_F16, 1, &head, nullptr, nullptr, 8, 1, nullptr, nullptr, nullptr, F, big,
                                 nullptr));
  rejected(moe_prerouter_forward(F, MOE_F16, 1, &head, nullptr, nullptr, 8, 1, FI, FF, nullptr, F, 64, nullptr));
  rejected(moe_prerouted_layer_forward(F, MOE_F16, 1, FF, &ex, 8, 1, FF, FI, FF, &head, FI, FF, F, big, nullptr));
  rejected(moe_prerouted_layer_forward(F, MOE_F16, 1, FF, &ex, 8, 1, FF, nullptr, FF, &head, nullptr, FF, F, big,
                                       nullptr));
  // quantized linear with a delta, quantiser, staging, remap, stream read, timer
  moe_qweight qw{2048, 2048, MOE_Q_INT4, F, FS};
  moe_qweight qbad{2048, 2040, MOE_Q_INT4, F, FS};
  rejected(moe_qlinear_lora_forward(F, MOE_F16, 1, &qbad, nullptr, nullptr, 0, 0.f, FF, F, big, nullptr));
  rejected(moe_qlinear_lora_forward(F, MOE_F16, 1, &qw, nullptr, nullptr, 4, 1.f, FF, F, big, nullptr));
  rejected(moe_qlinear_lora_forward(F, MOE_F16, 1, &qw, FF, FF, 65, 1.f, FF, F, big, nullptr));
  rejected(moe_quantize(FF, 4, 33, MOE_Q_SYM8, F, FS, nullptr));
  rejected(moe_quantize(FF, 4, 32, 3, F, FS, nullptr));
  const moe_experts stack_bad = experts(8, 1024, 512, MOE_Q_SYM8);
  rejected(moe_stage_experts(&ex, &stack_bad, FI, FI, 2, nullptr));
  rejected(moe_stage_experts(&ex, &ex, nullptr, FI, 2, nullptr));
  rejected(moe_remap_ids(nullptr, 4, FI, 256, FI, nullptr));
  rejected(moe_remap_ids(FI, -1, FI, 256, FI, nullptr));
  rejected(moe_stream_read(F, 1000, nullptr));
  rejected(moe_stream_read(MIS, 1024, nullptr));
  rejected(moe_timer_start(99, 4));
  rejected(moe_timer_start(0, 0));
  rejected(moe_timer_read(nullptr, 4, nullptr));

  // miss-policy replay on seeded routings, every policy, with and without admission
  std::mt19937 g(7);
  for (int rep = 0; rep < 24; ++rep) {
    const int E = 8 + (int)(g() % 505), k = 1 + (int)(g() % 10), T = (int)(g() % 200);
    const int C = k + (int)(g() % (E - k + 1));
    std::vector<int32_t> idx((size_t)T * k);
    std::vector<float> gate((size_t)T * k);
    for (int t = 0; t < T; ++t) {
      std::vector<int32_t> pool(E);
      for (int e = 0; e < E; ++e) pool[e] = e;
      float sum = 0;
      for (int s = 0; s < k; ++s) {
        const int j = s + (int)(g() % (E - s));
        std::swap(pool[s], pool[j]);
        idx[(size_t)t * k + s] = pool[s];
        gate[(size_t)t * k + s] = 1.0f / (1.0f + s);
        sum += gate[(size_t)t * k + s];
      }
      for (int s = 0; s < k; ++s) gate[(size_t)t * k + s] /= sum;
    }
    std::vector<float> m(T + 1);
    std::vector<int32_t> sync(T + 1), bg(T + 1);
    std::vector<uint8_t> res(E);
    for (int pol = 0; pol < 3; ++pol)
      for (float beta : {0.0f, 0.5f}) {
        CHECK(moe_miss_replay(idx.data(), gate.data(), T, k, E, C, pol, 0.15f, beta, m.data(), sync.data(), bg.data(),
                              res.data()) == MOE_OK);
        int resident = 0;
        for (int e = 0; e < E; ++e) resident += res[e];
        CHECK(resident <= C);
      }
    if (T > 0 && k > 1) {
      idx[1] = idx[0];  // an expert twice in one token
      rejected(moe_miss_replay(idx.data(), gate.data(), T, k, E, C, 0, 0.15f, 0.f, m.data(), sync.data(), bg.data(),
                               res.data()));
      idx[1] = E;  // out of range
      rejected(moe_miss_replay(idx.data(), gate.data(), T, k, E, C, 0, 0.15f, 0.f, m.data(), sync.data(), bg.data(),
                               res.data()));
    }
  }
  std::printf("ok\n");
  return 0;
}
