// Rank-64 instances of the fused LoRA / QLoRA input-gradient kernel of dx.hip.  They are
// compiled in this translation unit of their own, without the VGPR form for MFMAs that dx.hip
// is built with, because they accumulate through builtin MFMAs (the compiler tracks those
// results' latencies when it has to move accumulators between registers).
#define LORA_DX_RANK64_TU 1
#include "dx.hip"
