// Empty stand-in for the HIP runtime header in the host build of quantize.h (test only).
#pragma once
