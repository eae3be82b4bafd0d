// Registration functions of the compiled GEMV instances, one per translation
// unit; the host dispatch calls them once, in order (the first registered
// instance that takes a call's K is its default).
#pragma once

#include <vector>

#include "gemv_impl.h"

namespace skg {
void register_gemv_bf16(std::vector<GemvEntry>& out);
void register_gemv_q8_0_f32(std::vector<GemvEntry>& out);
void register_gemv_q8_0_f32_m38(std::vector<GemvEntry>& out);
void register_gemv_q4_0_f32(std::vector<GemvEntry>& out);
void register_gemv_q4_0_f32_m35(std::vector<GemvEntry>& out);
void register_gemv_q4_0_f32_m68(std::vector<GemvEntry>& out);
void register_gemv_q8_1(std::vector<GemvEntry>& out);
void register_gemv_mfma_q4_0(std::vector<GemvEntry>& out);
void register_gemv_mfma_q8_0(std::vector<GemvEntry>& out);
void register_gemv_mfma_q4_0_alt(std::vector<GemvEntry>& out);
void register_gemv_mfma_q8_0_alt(std::vector<GemvEntry>& out);
void register_gemv_q4_K(std::vector<GemvEntry>& out);
void register_gemv_q6_K(std::vector<GemvEntry>& out);
void register_gemv_mfma_q8_1(std::vector<GemvEntry>& out);
void register_gemv_mfma_q8_1_alt(std::vector<GemvEntry>& out);
}  // namespace skg
